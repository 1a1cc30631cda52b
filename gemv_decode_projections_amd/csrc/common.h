// Shared device helpers for the gfx950 projection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kWave = 64;

// Fragment geometry of v_mfma_f32_16x16x32_bf16 as the kernels use it:
//   A (16 x 32, weights): lane l holds row l % 16, k = 8 * (l / 16) + 0..7;
//   B (32 x 16, tokens):  lane l holds column l % 16, the same k slots;
//   C (16 x 16, fp32):    lane l holds column l % 16, rows 4 * (l / 16) + 0..3.
// A dot product is independent of the order of its k terms, so any k
// permutation shared by A and B gives the same sum; what matters is that the
// weight repack and the activation loads agree on it.
constexpr int kRowsPerBlock = 16;
constexpr int kStepK = 32;

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed BF16 bits (lo in bits 0..15), round to nearest,
// ties to even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}


// 12-bit weights (lossless; the report's round-5 format: the low byte of each
// BF16 weight kept raw, the sign and a 3-bit code for one of eight exponent
// values chosen per matrix). A lane's eight weights w0..w7 of an MFMA A
// fragment take 12 bytes: dword 0 the low bytes of w0..w3, dword 1 those of
// w4..w7, dword 2 byte i = n(w_i) | n(w_{i+4}) << 4 with n = sign << 3 | code.
// The code indexes a table of eight high-byte values (BF16 bits 14..8),
// bytes 0..3 in t0 and 4..7 in t1, so one byte permute maps four codes at
// once. Returns the eight BF16 weights in the A-operand layout (w_{2j} in
// the low half of dword j).
__device__ __forceinline__ u32x4 decode12(u32x3 v, uint32_t t0, uint32_t t1)
{
    const uint32_t qa = v.z & 0x0f0f0f0fu;
    const uint32_t qb = (v.z >> 4) & 0x0f0f0f0fu;
    const uint32_t ha = __builtin_amdgcn_perm(t1, t0, qa & 0x07070707u) | ((qa << 4) & 0x80808080u);
    const uint32_t hb = __builtin_amdgcn_perm(t1, t0, qb & 0x07070707u) | ((qb << 4) & 0x80808080u);
    return u32x4{__builtin_amdgcn_perm(ha, v.x, 0x05010400u), __builtin_amdgcn_perm(ha, v.x, 0x07030602u),
                 __builtin_amdgcn_perm(hb, v.y, 0x05010400u), __builtin_amdgcn_perm(hb, v.y, 0x07030602u)};
}

// BF16 bits -> FP32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __builtin_bit_cast(float, bits << 16); }

// Exact three-way split of eight FP32 weights into BF16 parts, w = hi + mid + lo.
// hi keeps the top 8 significand bits (truncation), mid the next 8 of the
// exact remainder, lo the last 8; each subtraction is exact because the
// subtrahend is a prefix of the minuend's significand, and the last remainder
// has at most 8 significant bits. Every product of a BF16 activation with a
// part is exact in FP32, so the MFMA sees the weight at full FP32 precision.
// (Values below 2^-103 in magnitude would lose bits to FP32 subnormals; the
// router's weights are many orders of magnitude above that.)
__device__ __forceinline__ void split3_f32(const u32x4 &w0, const u32x4 &w1, u32x4 &hi, u32x4 &mid,
                                           u32x4 &lo)
{
    uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t h[8], md[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t uh = w[e] & 0xffff0000u;
        float r1 = __builtin_bit_cast(float, w[e]) - __builtin_bit_cast(float, uh);
        uint32_t um = __builtin_bit_cast(uint32_t, r1) & 0xffff0000u;
        float r2 = r1 - __builtin_bit_cast(float, um);
        h[e] = uh;
        md[e] = um;
        l[e] = __builtin_bit_cast(uint32_t, r2);
    }
    // Pack pairs: element 2j in the low half, 2j+1 in the high half.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi[j] = (h[2 * j] >> 16) | (h[2 * j + 1] & 0xffff0000u);
        mid[j] = (md[2 * j] >> 16) | (md[2 * j + 1] & 0xffff0000u);
        lo[j] = (l[2 * j] >> 16) | (l[2 * j + 1] & 0xffff0000u);
    }
}

// Polled split-K over workgroups (the skinny kernel): the workspace
// holds every split's FP32 partial tile, and a 32-bit word with all bits set
// means "not written yet" (the library fills the workspace with that mark
// once; each reduction puts it back). One split per tile, the one the
// hardware dispatches last, reduces: it polls the others' words with loads
// that bypass the XCD-local L2 until none holds the mark. The other splits
// only publish and exit, so no arrival counter, store acknowledgement or
// cache flush is needed.
constexpr uint32_t kEmptyWord = 0xffffffffu;
// A reducer gives up after kPollLimit polls of a word (about a quarter of a
// second): the missing words then read as NaN, so a launch always ends and a
// lost partial shows in the output; the reducer also counts the give-up in a
// per-layer word the host can read. Only a split held off the chip for that
// long could publish after its reducer gave up, leaving words that a later
// launch on the same layer would read as arrived; the host's reset of the
// count restores every mark.
constexpr int kPollLimit = 1 << 18;

// The one NaN pattern that equals the mark is published as the default NaN.
__device__ __forceinline__ uint32_t publishable(uint32_t u) { return u == kEmptyWord ? 0x7fc00000u : u; }
__device__ __forceinline__ u32x4 publishable(u32x4 u)
{
    return u32x4{publishable(u.x), publishable(u.y), publishable(u.z), publishable(u.w)};
}

// Index, among the n logical workgroup ids l0, l0 + stride, ..., of the one
// with the highest hardware id: the reducer of a tile. Dispatch runs in
// hardware-id order, so every workgroup the reducer waits for has been
// placed on the chip before it and finishes without waiting itself. With the
// XCD remap (G % 8 == 0) logical id l runs on hardware id
// 8 * (l % (G / 8)) + l / (G / 8); the walk uses one division.
__host__ __device__ __forceinline__ int reducing_split(int l0, int stride, int n, int G, bool remap)
{
    if (!remap)
        return n - 1;
    const int per = G / 8;
    int q = l0 / per, r = l0 - q * per, best = -1, rs = n - 1;
    for (int s = 0; s < n; ++s) {
        if (8 * r + q > best) {
            best = 8 * r + q;
            rs = s;
        }
        r += stride;
        while (r >= per) {
            r -= per;
            ++q;
        }
    }
    return rs;
}

}  // namespace gdp
