// Prepare-time weight repack: N x K row-major -> fragment-major.
//
// A lossless reordering of W into the order the kernels read it, done once
// before any timed call (guide ch. 1 "The problem, the judge and the speed of
// light", §1.6: prepare repacks the weights; the notebook's packed-pooler
// notes store W tile-major in the kernel's read order).
//
// Packed order, BF16: [N/16 row blocks][K/32 k-steps][64 lanes][8 values]:
// the 16-byte unit of lane l in fragment (rb, s) holds W[rb*16 + l%16]
// [s*32 + 8*(l/16) + 0..7], the A-operand slot of v_mfma_f32_16x16x32_bf16.
// FP32 (router): [N/16][K/32][2 halves][64 lanes][4 values]: half h of lane
// l holds W[rb*16 + l%16][s*32 + 8*(l/16) + 4h + 0..3], so each 16-byte load
// of a wave is 1 KB contiguous.
// Row block rb occupies one contiguous span, so the first 1024 rows of the
// unpooler (its slice at <= 8 tokens) are a contiguous prefix.
#pragma once

#include "common.h"

namespace gdp {

__global__ void repack_bf16_kernel(const uint16_t *__restrict__ W, u32x4 *__restrict__ out, int N, int K)
{
    const int KS = K / kStepK;
    const size_t units = (size_t)N * K / 8;
    for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const size_t frag = u / kWave;
        const int s = (int)(frag % KS);
        const size_t rb = frag / KS;
        const size_t row = rb * kRowsPerBlock + lane % 16;
        const size_t k0 = (size_t)s * kStepK + 8 * (lane / 16);
        out[u] = *reinterpret_cast<const u32x4 *>(W + row * K + k0);
    }
}

__global__ void repack_f32_kernel(const float *__restrict__ W, u32x4 *__restrict__ out, int N, int K)
{
    const int KS = K / kStepK;
    const size_t units = (size_t)N * K / 4;
    for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const int half = (int)((u / kWave) % 2);
        const size_t frag = u / (2 * kWave);
        const int s = (int)(frag % KS);
        const size_t rb = frag / KS;
        const size_t row = rb * kRowsPerBlock + lane % 16;
        const size_t k0 = (size_t)s * kStepK + 8 * (lane / 16) + 4 * half;
        out[u] = *reinterpret_cast<const u32x4 *>(W + row * K + k0);
    }
}

// 12-bit packing (decode12 in common.h): the same fragment order as the BF16
// repack, 12 bytes per lane unit: [N/16][K/32][64 lanes][12 bytes]. Weights
// whose exponent byte is outside the table (base .. base+7 for bits 14..8)
// are stored with the nearest table code; the exact weight is restored by a
// per-row correction list built on the host (proj_prepare).
__global__ void repack_z_kernel(const uint16_t *__restrict__ W, uint32_t *__restrict__ out, int N, int K, int base)
{
    const int KS = K / kStepK;
    const size_t units = (size_t)N * K / 8;
    for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const size_t frag = u / kWave;
        const int s = (int)(frag % KS);
        const size_t rb = frag / KS;
        const size_t row = rb * kRowsPerBlock + lane % 16;
        const size_t k0 = (size_t)s * kStepK + 8 * (lane / 16);
        const u32x4 src = *reinterpret_cast<const u32x4 *>(W + row * K + k0);
        uint32_t lo[2] = {0u, 0u}, q = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w = (src[i / 2] >> (16 * (i % 2))) & 0xffffu;
            const int h = (int)((w >> 8) & 0x7fu);
            const uint32_t c = (uint32_t)min(max(h - base, 0), 7);
            const uint32_t n = ((w >> 15) << 3) | c;
            lo[i / 4] |= (w & 0xffu) << (8 * (i % 4));
            q |= n << (8 * (i % 4) + 4 * (i / 4));
        }
        out[3 * u + 0] = lo[0];
        out[3 * u + 1] = lo[1];
        out[3 * u + 2] = q;
    }
}

}  // namespace gdp
