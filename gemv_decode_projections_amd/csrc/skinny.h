// Skinny MFMA kernel: out = x @ W^T for a few tokens, weights streamed once.
//
// The operation and its regime come from guide ch. 1 "The problem, the judge
// and the speed of light" (§1.1 the layer, §1.7: at these token counts the
// work is a stream of weight bytes with little math attached). The report
// "Muse Spark Open Kernel Challenge - muse_bf16_proj" (What did not pay off;
// Rounds 3 and 5) found that splitting K between the warps of one block beat
// a cross-block reduction and that the next batch of weight loads must be in
// flight while the current one is multiplied; both carry over here.
//
// gfx950 design:
//   * W is pre-packed in fragment-major order (see repack.h): for each
//     16-row block, K/32 fragments of 1 KB (BF16) or 2 KB (FP32), each one
//     exactly the A operand of v_mfma_f32_16x16x32_bf16 for 64 lanes. A wave
//     therefore reads 1 KB contiguous per 16-byte-per-lane load.
//   * A workgroup owns RB row blocks, NT*16 tokens and a K range; its WAVES
//     waves split that K range into contiguous runs of SPW k-steps.
//   * Activations are the B operand, loaded straight from x (L2-resident
//     after the first touch) with quad-contiguous reads and permuted across
//     lanes into the MFMA layout; lanes of tokens >= m are zeroed.
//   * Loads are double-buffered in registers in stages of U k-steps; each
//     wave starts its run at a rotated k-step (spreads activation requests
//     over L2 channels).
//   * The waves' partial 16x16 tiles are summed through LDS in wave order.
//   * With KSPLIT > 1 one workgroup of each tile, the one the hardware
//     dispatches last, reduces; the others write their FP32 partials to a
//     workspace with cache-coherent atomic stores and exit. The reducer polls
//     those words until none holds the empty mark (all bits set), sums the
//     partials in split order with its own in place (deterministic), stores
//     the output and puts the mark back for the next launch.
//   * FP32 router weights are split exactly into three BF16 parts in
//     registers (common.h) and accumulated by three MFMAs in FP32.
//   * Z: weights read in the 12-bit lossless form (common.h, decode12; the
//     report's round 5 found 25 % fewer bytes worth ~20 % of a decode GEMV):
//     12 bytes per lane per fragment (one dwordx3 load, a wave's 768 bytes
//     contiguous), decoded with byte permutes right before the MFMA. Weights
//     outside the exponent table are corrected from a per-row list of
//     (k, w, d) with d the value the 12-bit form decodes to: one extra wave
//     loads the workgroup's list and gathers the activations it needs while
//     the other waves stream, and the epilogue applies (acc - d*x) + w*x in
//     list order (both products exact in FP32, so a one-hot activation row
//     returns the original weight bit for bit).
#pragma once

#include <type_traits>

#include "common.h"

namespace gdp {

struct SkinnyArgs {
    const void *wp;          // packed weights
    const uint16_t *x;       // m x K BF16
    void *out;               // m x n_eff (BF16 or FP32)
    uint64_t *pws;           // split-K partials; every word all ones between launches
    int m;
    int K;
    int n_eff;
    int n_rt;                // row tiles (n_eff / (16 * RB))
    int n_tt;                // token tiles (ceil(m / (16 * NT)))
    int ksplit;              // workgroups per tile along K
    int xcd_remap;           // 1: spread consecutive logical tiles on one XCD
    uint32_t *giveups;       // split-K: incremented once per reducer wave that stops waiting
    int poll_limit;          // split-K: polls of a word before the reducer stops waiting
    int drop_publish;        // test only: splits that do not reduce exit without publishing
    // 12-bit weights (Z variants only)
    const uint32_t *wz;      // packed 12-bit fragments
    uint32_t wz_bytes;
    uint32_t zt0, zt1;       // exponent table (high bytes), codes 0..3 and 4..7
    int zcr;                 // correction slots per row (0: none)
    const uint64_t *zexc;    // per row zcr slots: k | w << 16 | d << 32 (k = 0xffff: empty)
};

constexpr int kZMaxSlots = 8;    // correction slots per row a 12-bit layer may use
constexpr int kSkMaxParts = 4;   // stream partition: most shares covering one row block

// XP > 0: at most XP (4 or 8) tokens; each wave loads its whole activation
// slice (XP rows x SPW k-steps) into registers once instead of one 16-byte
// load per lane and k-step, and takes every k-step's B fragment from those
// registers with lane permutes. At <= 8 tokens a per-k-step load moves 1 KB
// per wave for at most 8 rows x 64 useful bytes; dropping them measured
// 0.7-2.1 us on the 8192-wide layers at one token.
// SKM: stream partition. The layer's (16-row block, k-step) pairs, in the
// packing's own order (row block major), are dealt in equal contiguous shares
// of WAVES * SPW to the workgroups, so every compute unit streams the same
// number of weight bytes whatever the layer's row count. A share spans the
// end of one row block (segment A) and possibly the start of the next (B);
// the kernel is then instantiated with RB = 2, one accumulator tile per
// segment, and each k-step feeds its one weight fragment to the accumulator
// of its own segment. A row block is covered by one to kSkMaxParts shares;
// their partials are summed by the one the hardware dispatched last (as in
// the polled split-K).
template <int NT, int RB, int WAVES, int SPW, bool F32W, bool Z = false, int XP = 0, bool SKM = false>
__global__ __launch_bounds__((WAVES + (Z ? 1 : 0)) * kWave) void skinny_kernel(SkinnyArgs a)
{
    static_assert(!(Z && F32W), "12-bit weights are BF16 only");
    static_assert(!SKM || (RB == 2 && !F32W && XP == 0), "stream partition: two segments, BF16 weights");
    static_assert(XP == 0 || ((XP == 4 || XP == 8) && NT == 1 && !F32W), "preloaded activations: 4 or 8 rows, one token block");
    static_assert(!Z || WAVES > 1, "12-bit variants need a separate wave for the corrections");
    constexpr int U = SPW < 4 ? SPW : 4;             // k-steps per pipeline stage
    static_assert(SPW % U == 0, "SPW must be a multiple of the stage size");
    constexpr int NSTAGE = SPW / U;
    constexpr int AW = F32W ? 2 : 1;                 // 16-byte loads per A fragment
    constexpr int FRAG_U4 = AW * kWave;              // u32x4 per fragment

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;

    // Workgroup -> (row tile, split, token tile). With xcd_remap, the 8
    // consecutive hardware ids that land on 8 different XCDs are turned into
    // logical ids that stay on one XCD, so token tiles of one row tile share
    // that XCD's L2.
    const int G = gridDim.x;
    int L = blockIdx.x;
    if (a.xcd_remap)
        L = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    const int tt = L % a.n_tt;
    const int rest = L / a.n_tt;
    const int ks = rest % a.ksplit;
    const int rt = rest / a.ksplit;

    // Split-K reducer of this tile (used after the main loop, computed here
    // off the critical path).
    const int rs = a.ksplit > 1 ? reducing_split(rt * a.ksplit * a.n_tt + tt, a.n_tt, a.ksplit, G, a.xcd_remap)
                                : 0;

    const int KS = a.K / kStepK;                     // k-steps in the whole row
    const int step0 = (ks * WAVES + wave) * SPW;     // this wave's first k-step
    // SKM: this workgroup's share [u0, u0 + WAVES * SPW) of the (row block,
    // k-step) units; unit v is k-step v - rb * KS of row block rb = v / KS,
    // and the packed fragment index is v itself.
    const int u0 = SKM ? L * (WAVES * SPW) : 0;
    const int rbA = SKM ? u0 / KS : 0;               // row block of segment A
    const int baseB = (rbA + 1) * KS;                // first unit of segment B
    const int vw = u0 + wave * SPW;                  // this wave's first unit
    const int rb0 = SKM ? rbA : rt * RB;

    const u32x4 *wbase = reinterpret_cast<const u32x4 *>(a.wp);
    // Each wave walks its k-steps starting at a rotated position, so waves of
    // one workgroup and neighbouring workgroups on an XCD do not all request
    // the same activation lines (and L2 channel) at the same moment.
    const int rot = SKM ? 0 : (2 * (wave + WAVES * (int)(blockIdx.x / 8))) & (SPW - 1);
    static_assert(SKM || (SPW & (SPW - 1)) == 0, "SPW must be a power of two");

    // Activations. The MFMA wants lane l to hold token l%16, k = 8*(l/16)+0..7,
    // which as a load would make every lane quad touch four rows (measured
    // ~3x slower than quad-contiguous reads from L2). So lane s loads token
    // s/4, k = 8*(s%4)+0..7 -- each quad one contiguous 64-byte row segment --
    // and the fragment is moved to the MFMA layout with a lane permutation
    // (destination lane l takes source lane 4*(l%16) + l/16).
    bool tok_ok[NT];
    const uint16_t *xrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int tok = tt * 16 * NT + t * 16 + (lane % 16);       // this lane's MFMA column
        tok_ok[t] = tok < a.m;
        const int tok_ld = tt * 16 * NT + t * 16 + lane / 4;       // the row this lane loads
        // Rows past the last token read row m-1 (always valid); their lanes are
        // zeroed after the permutation. A select instead of a branch keeps the
        // load pipeline free of control-flow joins, which force a full wait.
        xrow[t] = a.x + (size_t)(tok_ld < a.m ? tok_ld : a.m - 1) * a.K + 8 * (lane % 4);
    }
    const int perm_src = 4 * (lane % 16) + lane / 16;             // bpermute source lane

    // Preloaded activations (XP > 0): register j of lane L holds the k-step
    // the loop visits j * KPR + L / (4 XP)-th (the wave's run in its rotated
    // order), token row (L % (4 XP)) / 4, k-group L % 4 (each lane quad one
    // contiguous 64-byte row segment, as above). The B fragment of the s-th
    // visited k-step (token l % 16, k-group l / 16) is then lane
    // (s % KPR) * 4 XP + 4 (l % 16) + l / 16 of register s / KPR: one
    // register index for the whole wave, known at compile time.
    constexpr int KPR = XP ? 16 / XP : 1;                        // k-steps per register
    constexpr int NXR = XP ? SPW / KPR : 1;                       // registers per lane
    static_assert(XP == 0 || SPW % KPR == 0, "whole registers of k-steps");
    u32x4 xp[NXR];
    int xsrc[KPR];
#pragma unroll
    for (int q = 0; q < KPR; ++q)
        xsrc[q] = (XP && lane % 16 < XP) ? q * 4 * XP + 4 * (lane % 16) + lane / 16 : 0;

    f32x4 acc[RB][NT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wa[2][U][RB][AW];
    u32x3 wq[2][U][RB];
    u32x4 xb[2][U][NT];
    // Buffer descriptor over the 12-bit weights (built but unused when !Z).
    const __amdgpu_buffer_rsrc_t wzr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.wz), (short)0, (int)a.wz_bytes, 0x00020000);

    // Plain (cached) loads: measured faster than non-temporal ones for the
    // weight stream on this part.
    auto load_stage = [&](int buf, int local) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int step = step0 + ((local + u + rot) & (SPW - 1));
            if constexpr (SKM) {
                const int v = vw + local + u;
                step = v - (v >= baseB ? baseB : baseB - KS);
                if constexpr (Z)
                    wq[buf][u][0] = __builtin_amdgcn_raw_buffer_load_b96(wzr, (uint32_t)((v * kWave + lane) * 12), 0, 0);
                else
                    wa[buf][u][0][0] = wbase[(size_t)v * FRAG_U4 + lane];
            }
#pragma unroll
            for (int r = 0; r < (SKM ? 0 : RB); ++r) {
                if constexpr (Z) {
                    wq[buf][u][r] = __builtin_amdgcn_raw_buffer_load_b96(
                        wzr, (uint32_t)((((rb0 + r) * KS + step) * kWave + lane) * 12), 0, 0);
                } else {
                    const u32x4 *f = wbase + ((size_t)(rb0 + r) * KS + step) * FRAG_U4 + lane;
#pragma unroll
                    for (int h = 0; h < AW; ++h)
                        wa[buf][u][r][h] = f[h * kWave];
                }
            }
            if constexpr (XP == 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    xb[buf][u][t] = *reinterpret_cast<const u32x4 *>(xrow[t] + step * kStepK);
            }
        }
        // Keep a stage's loads where they are issued: the scheduler otherwise
        // sinks them toward their first use, leaving 2-5 k-steps in flight
        // per wave instead of 4-8 (cold sweeps: qkv_gate and the unpooler
        // 0.3 us faster at 1-16 tokens, the pooler 1.2 us at 32). Waves that
        // run a single stage (the router's) measured slower with it.
        if constexpr (NSTAGE > 1 && !F32W)
            __builtin_amdgcn_sched_barrier(0);
    };

    auto compute_stage = [&](int buf, int local) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                u32x4 v;
                if constexpr (XP) {
                    const int s = local + u;              // compile-time once the stages are unrolled
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc[s % KPR] * 4, (int)xp[s / KPR][i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_src * 4, (int)xb[buf][u][t][i]);
                }
                xb[buf][u][t] = tok_ok[t] ? v : u32x4{0u, 0u, 0u, 0u};
            }
            if constexpr (SKM) {
                // One fragment per k-step, into the accumulator of its segment
                // (the other MFMA multiplies zeros: the MFMA units idle here).
                const bool segA = vw + local + u < baseB;
                const u32x4 wf = Z ? decode12(wq[buf][u][0], a.zt0, a.zt1) : wa[buf][u][0][0];
                const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    acc[0][t] = mfma16x16x32(wf, segA ? xb[buf][u][t] : zero, acc[0][t]);
                    acc[1][t] = mfma16x16x32(wf, segA ? zero : xb[buf][u][t], acc[1][t]);
                }
            }
#pragma unroll
            for (int r = 0; r < (SKM ? 0 : RB); ++r) {
                if constexpr (F32W) {
                    u32x4 hi, mid, lo;
                    split3_f32(wa[buf][u][r][0], wa[buf][u][r][1], hi, mid, lo);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        acc[r][t] = mfma16x16x32(hi, xb[buf][u][t], acc[r][t]);
                        acc[r][t] = mfma16x16x32(mid, xb[buf][u][t], acc[r][t]);
                        acc[r][t] = mfma16x16x32(lo, xb[buf][u][t], acc[r][t]);
                    }
                } else {
                    const u32x4 wf = Z ? decode12(wq[buf][u][r], a.zt0, a.zt1) : wa[buf][u][r][0];
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[r][t] = mfma16x16x32(wf, xb[buf][u][t], acc[r][t]);
                }
            }
        }
    };

    // 12-bit corrections: this workgroup's rows' slots (zcr per row; row r's
    // slot c at r * kZMaxSlots + c here), each with its weight pair and the
    // activations of the tile's tokens at k, and per row a byte mask of the
    // slots that are live in this split (entry present, k in its range).
    constexpr int ZSLOTS = Z ? 16 * RB * kZMaxSlots : 1;
    constexpr int ZTOK = 16 * NT;
    __shared__ __attribute__((aligned(16))) float zw[ZSLOTS], zd[ZSLOTS];
    __shared__ float zx[ZSLOTS][Z ? ZTOK : 1];
    __shared__ __attribute__((aligned(8))) uint8_t zlive[ZSLOTS];
    __shared__ uint32_t zlist[ZSLOTS];               // live slots: slot | k << 16
    const bool exc_wave = Z && wave == WAVES;

    if (exc_wave) {
        if constexpr (Z) {
          if (a.zcr > 0) {
            // The slot entries are loaded at once; the live ones (about one
            // per row) are packed into a list, and the activations are
            // gathered for (live slot, token) pairs only, a batch of loads
            // per lane in flight at a time.
            constexpr int EPL = ZSLOTS / kWave;       // slots per lane (at the maximum)
            // SKM: rows 0-15 are segment A (k from the share's start to the
            // row block's end), rows 16-31 segment B (k from 0), present
            // only when the share reaches the next row block.
            const int skB = SKM ? max(0, u0 + WAVES * SPW - baseB) : 0;     // units of segment B
            const int nslot = (SKM ? (skB > 0 ? 32 : 16) : 16 * RB) * a.zcr;
            const uint64_t *src = a.zexc + (size_t)rb0 * 16 * a.zcr;
            const int k_lo = SKM ? (u0 - (baseB - KS)) * kStepK : (ks * WAVES) * SPW * kStepK;
            const int k_hi = SKM ? min(KS, u0 - (baseB - KS) + WAVES * SPW) * kStepK : k_lo + WAVES * SPW * kStepK;
            const int ntok = min(a.m - tt * ZTOK, ZTOK);   // live tokens of this tile
            uint64_t ent[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                ent[i] = src[min(lane + kWave * i, nslot - 1)];
            int nlive = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int j = lane + kWave * i;
                const int k = (int)(ent[i] & 0xffffu);
                const int r = j / a.zcr, c = j - (j / a.zcr) * a.zcr;
                const bool live = j < nslot && (SKM && r >= 16 ? k < skB * kStepK : k >= k_lo && k < k_hi);
                const int sl = r * kZMaxSlots + c;
                if (j < nslot) {
                    zlive[sl] = live ? 1 : 0;
                    zw[sl] = bf16_to_f32((uint32_t)(ent[i] >> 16) & 0xffffu);
                    zd[sl] = bf16_to_f32((uint32_t)(ent[i] >> 32) & 0xffffu);
                }
                const uint64_t mask = __ballot(live);
                if (live)
                    zlist[nlive + __popcll(mask & ((1ull << lane) - 1ull))] = (uint32_t)sl | ((uint32_t)k << 16);
                nlive += __popcll(mask);
            }
            // Slots past zcr in each row stay dead.
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int sl = lane + kWave * i;
                if ((sl % kZMaxSlots) >= a.zcr)
                    zlive[sl] = 0;
            }
            // One wave wrote the list; make its LDS writes visible to its own
            // later reads from other lanes.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            constexpr int G = 8;                      // gathers in flight per lane
            const int pairs = nlive * ntok;
            const uint16_t *xt = a.x + (size_t)tt * ZTOK * a.K;
            for (int p0 = 0; p0 < pairs; p0 += G * kWave) {
                uint32_t v[G], dst[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int p = min(p0 + g * kWave + lane, pairs - 1);
                    const int e = p / ntok, t = p - (p / ntok) * ntok;
                    const uint32_t le = zlist[e];
                    dst[g] = (le & 0xffffu) * ZTOK + t;
                    v[g] = xt[(size_t)t * a.K + (le >> 16)];
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if (p0 + g * kWave + lane < pairs)
                        (&zx[0][0])[dst[g]] = bf16_to_f32(v[g]);
            }
          }
        }
    } else {
        if constexpr (XP) {
            const int row = (lane % (4 * XP)) / 4;
            const int tok = tt * 16 + row;
            const uint16_t *xr = a.x + (size_t)(tok < a.m ? tok : a.m - 1) * a.K + 8 * (lane % 4);
#pragma unroll
            for (int j = 0; j < NXR; ++j)
                xp[j] = *reinterpret_cast<const u32x4 *>(
                    xr + (size_t)(step0 + ((j * KPR + lane / (4 * XP) + rot) & (SPW - 1))) * kStepK);
        }
        load_stage(0, 0);
        if constexpr (NSTAGE > 1)
            load_stage(1, U);
#pragma unroll
        for (int s = 0; s < NSTAGE; s += 2) {
            compute_stage(0, s * U);
            if (s + 2 < NSTAGE)
                load_stage(0, (s + 2) * U);
            if (s + 1 < NSTAGE) {
                compute_stage(1, (s + 1) * U);
                if (s + 3 < NSTAGE)
                    load_stage(1, (s + 3) * U);
            }
        }
    }

    // Sum the waves' partial tiles in wave order.
    constexpr int TILES = RB * NT;
    constexpr int ELEMS = TILES * kWave;             // f32x4 per workgroup tile
    __shared__ f32x4 red[WAVES > 1 ? WAVES : 1][TILES][kWave];
    if constexpr (WAVES > 1) {
        if (!exc_wave) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    red[wave][r * NT + t][lane] = acc[r][t];
        }
        __syncthreads();
    }

    const int tile = rt * a.n_tt + tt;

    // 12-bit corrections, applied once per (row, token) by its own thread
    // (the pairs are spread over the whole workgroup): zfin = sum of the
    // waves' partials in wave order, then for each live slot of the row in
    // slot order v = (v - d*x) + w*x.
    constexpr int ZROWS = 16 * RB;
    __shared__ float zfin[Z ? ZROWS : 1][Z ? ZTOK : 1];
    if constexpr (Z && WAVES > 1) {
        if (a.zcr > 0) {
            for (int p = threadIdx.x; p < ZROWS * ZTOK; p += (WAVES + 1) * kWave) {
                const int row = p / ZTOK, tl = p % ZTOK;
                const int r = row / kRowsPerBlock, rr = row % kRowsPerBlock;
                const int j = r * NT + tl / 16;
                const int ln = 16 * (rr / 4) + tl % 16;
                float v = reinterpret_cast<const float *>(&red[0][j][ln])[rr % 4];
#pragma unroll
                for (int w = 1; w < WAVES; ++w)
                    v += reinterpret_cast<const float *>(&red[w][j][ln])[rr % 4];
                if (tt * ZTOK + tl < a.m) {
                    // All of the row's slots are read at once and the dead
                    // ones skipped by a select, so the reads overlap instead
                    // of forming a chain one slot long each.
                    const int s0 = row * kZMaxSlots;
                    const uint64_t live = *reinterpret_cast<const uint64_t *>(&zlive[s0]);
                    const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&zd[s0]);
                    const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&zd[s0 + 4]);
                    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&zw[s0]);
                    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&zw[s0 + 4]);
                    float xs[kZMaxSlots];
#pragma unroll
                    for (int c = 0; c < kZMaxSlots; ++c)
                        xs[c] = zx[s0 + c][tl];
#pragma unroll
                    for (int c = 0; c < kZMaxSlots; ++c) {
                        const float d = c < 4 ? d0[c % 4] : d1[c % 4];
                        const float w = c < 4 ? w0[c % 4] : w1[c % 4];
                        const float u = (v - d * xs[c]) + w * xs[c];
                        v = ((live >> (8 * c)) & 1u) ? u : v;
                    }
                }
                zfin[row][tl] = v;
            }
            __syncthreads();
        }
    }

    // Sum of the waves' partials for element e (with the 12-bit corrections
    // when there are any).
    auto wave_sum = [&](int e) -> f32x4 {
        if constexpr (WAVES > 1) {
            if constexpr (Z) {
                if (a.zcr > 0) {
                    const int j = e / kWave, ln = e % kWave;
                    const int r = j / NT, t = j % NT;
                    const int tl = t * 16 + (ln % 16);
                    const int row0 = r * kRowsPerBlock + 4 * (ln / 16);
                    return f32x4{zfin[row0][tl], zfin[row0 + 1][tl], zfin[row0 + 2][tl], zfin[row0 + 3][tl]};
                }
            }
            f32x4 v = red[0][e / kWave][e % kWave];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                v += red[w][e / kWave][e % kWave];
            return v;
        } else {
            return f32x4{0.f, 0.f, 0.f, 0.f};  // never called with one wave
        }
    };

    auto store_out = [&](int e, f32x4 v) {
        const int j = e / kWave, ln = e % kWave;
        const int r = j / NT, t = j % NT;
        const int tk = tt * 16 * NT + t * 16 + (ln % 16);
        if (tk >= a.m)
            return;
        const int row = (rb0 + r) * kRowsPerBlock + 4 * (ln / 16);
        if constexpr (F32W) {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + (size_t)tk * a.n_eff + row) = v;
        } else {
            u32x2 p;
            p.x = pack_bf16x2(v.x, v.y);
            p.y = pack_bf16x2(v.z, v.w);
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + (size_t)tk * a.n_eff + row) = p;
        }
    };

    // With WAVES == 1 only the owning lane may read its accumulators.
    constexpr int NTHR = (WAVES + (Z ? 1 : 0)) * kWave;
    if constexpr (SKM) {
        // Per segment: the shares covering its row block are first..last
        // (consecutive logical ids); alone, the share stores the output;
        // otherwise the one dispatched last sums the parts in share order
        // (its own from the wave sum), the others publish and move on. A
        // share waits only on shares with lower hardware ids, which are on
        // the chip before it, so no wait is circular.
        // Every publish comes before any wait (two passes over the
        // segments): a share that reduced first and published after would
        // make the next share's reduction wait for its reduction, and so on
        // down the grid.
        constexpr int SE = NT * kWave;                  // f32x4 per segment tile
        constexpr uint64_t kEmpty = ~0ull;
        const int P = WAVES * SPW;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const int rb = rbA + sg;
            if (max(rb * KS, u0) >= min((rb + 1) * KS, u0 + P))
                continue;                               // the share does not reach this row block
            const int first = (rb * KS) / P, last = ((rb + 1) * KS - 1) / P;
            const int nparts = last - first + 1, slot = L - first;
            const int rsg = nparts == 1 ? slot : reducing_split(first, 1, nparts, G, a.xcd_remap != 0);
            if ((slot == rsg) != (pass == 1))
                continue;                               // pass 0: publish; pass 1: store or reduce
            if (nparts == 1) {
                for (int e = threadIdx.x; e < SE; e += NTHR)
                    store_out(sg * SE + e, wave_sum(sg * SE + e));
                continue;
            }
            uint64_t *parts = a.pws + (size_t)rb * kSkMaxParts * SE * 2;   // slot p: SE units of two words
            if (slot != rsg) {
                if (!a.drop_publish)
                    for (int e = threadIdx.x; e < SE; e += NTHR) {
                        const u32x4 u = publishable(__builtin_bit_cast(u32x4, wave_sum(sg * SE + e)));
                        uint64_t *d = parts + ((size_t)slot * SE + e) * 2;
                        __hip_atomic_store(d, (uint64_t)u.x | ((uint64_t)u.y << 32), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(d + 1, (uint64_t)u.z | ((uint64_t)u.w << 32), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    }
                continue;
            }
            for (int e0 = 0; e0 < SE; e0 += NTHR) {
                const int e = e0 + (int)threadIdx.x;
                const bool mine = e < SE;
                // Every other part's two words at once, then the ones still
                // empty again, bounded as in the polled split-K.
                uint64_t w[kSkMaxParts][2];
#pragma unroll
                for (int q = 0; q < kSkMaxParts; ++q)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        w[q][h] = (mine && q < nparts && q != slot)
                                      ? __hip_atomic_load(parts + ((size_t)q * SE + e) * 2 + h, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT)
                                      : 0ull;
                for (int poll = 0;; ++poll) {
                    bool miss = false;
#pragma unroll
                    for (int q = 0; q < kSkMaxParts; ++q)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            miss |= w[q][h] == kEmpty;
                    if (!__any(miss))
                        break;
                    if (poll >= a.poll_limit) {
#pragma unroll
                        for (int q = 0; q < kSkMaxParts; ++q)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                w[q][h] = w[q][h] == kEmpty ? 0x7fc000007fc00000ull : w[q][h];
                        if (lane == 0)
                            __hip_atomic_fetch_add(a.giveups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
#pragma unroll
                    for (int q = 0; q < kSkMaxParts; ++q)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            if (w[q][h] == kEmpty)
                                w[q][h] = __hip_atomic_load(parts + ((size_t)q * SE + e) * 2 + h, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                }
                if (mine) {
                    const f32x4 own = wave_sum(sg * SE + e);
                    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < kSkMaxParts; ++q) {
                        if (q >= nparts)
                            break;
                        if (q == slot) {
                            v += own;
                            continue;
                        }
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            __hip_atomic_store(parts + ((size_t)q * SE + e) * 2 + h, kEmpty, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        const u32x4 u = {(uint32_t)w[q][0], (uint32_t)(w[q][0] >> 32), (uint32_t)w[q][1],
                                         (uint32_t)(w[q][1] >> 32)};
                        v += __builtin_bit_cast(f32x4, u);
                    }
                    store_out(sg * SE + e, v);
                }
            }
        }
        return;
    }
    if (a.ksplit == 1) {
        if constexpr (WAVES > 1) {
            for (int e = threadIdx.x; e < ELEMS; e += NTHR)
                store_out(e, wave_sum(e));
        } else {
#pragma unroll
            for (int j = 0; j < TILES; ++j)
                store_out(j * kWave + lane, acc[j / NT][j % NT]);
        }
        return;
    }

    // Cross-workgroup split (common.h: polled partials, reducer = the split
    // dispatched last). The other splits publish their partial tile (8-byte
    // words, an f32x4 is two words, low element first) with agent-scope
    // atomic stores, which the compiler maps to cache-coherent write-through
    // accesses on this multi-XCD part, and exit. The reducer gathers WAVES
    // splits per round, one per wave: once one word of the split has arrived
    // it loads them all at once, re-reads the words still empty, marks every
    // word empty again, and sums through LDS in split order, taking its own
    // partial from registers at its place. The poll is bounded: after
    // a.poll_limit rounds the missing words count as NaN, so a launch always
    // ends (and a lost partial shows in the output and in the give-up count).
    constexpr int EPT = (ELEMS + NTHR - 1) / NTHR;  // output elements per thread
    constexpr uint64_t kEmpty = ~0ull;              // two empty words
    uint64_t *wsw = a.pws + (size_t)tile * a.ksplit * ELEMS * 2;
    if (ks != rs) {
        if (a.drop_publish)
            return;
        for (int e = threadIdx.x; e < ELEMS; e += NTHR) {
            const u32x4 u = publishable(__builtin_bit_cast(u32x4, wave_sum(e)));
            uint64_t *d = wsw + ((size_t)ks * ELEMS + e) * 2;
            __hip_atomic_store(d, (uint64_t)u.x | ((uint64_t)u.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(d + 1, (uint64_t)u.z | ((uint64_t)u.w << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    f32x4 own[EPT];
    f32x4 v[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * NTHR;
        own[i] = e < ELEMS ? wave_sum(e) : f32x4{0.f, 0.f, 0.f, 0.f};
        v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < a.ksplit; s0 += WAVES) {
        const int sp = s0 + wave;
        __syncthreads();                             // earlier readers of red are done
        if (!exc_wave && sp < a.ksplit && sp != rs) {
            uint64_t *src = wsw + (size_t)sp * ELEMS * 2;
            // Wait on one word first (one request per wave and round), so
            // that waiting reducers add little traffic to the streams of the
            // splits still running; then read all and re-read stragglers.
            int poll = 0;
            while (__hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kEmpty && poll < a.poll_limit)
                ++poll;
            uint64_t wd[TILES][2];
#pragma unroll
            for (int j = 0; j < TILES; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wd[j][h] = __hip_atomic_load(src + (j * kWave + lane) * 2 + h, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            for (;; ++poll) {
                bool miss = false;
#pragma unroll
                for (int j = 0; j < TILES; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        miss |= wd[j][h] == kEmpty;
                if (!__any(miss))
                    break;
                if (poll >= a.poll_limit) {
#pragma unroll
                    for (int j = 0; j < TILES; ++j)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            wd[j][h] = wd[j][h] == kEmpty ? 0x7fc000007fc00000ull : wd[j][h];
                    // Visible to the host (proj_split_giveups); the marks of
                    // this split are restored below like those of a complete one.
                    if (lane == 0)
                        __hip_atomic_fetch_add(a.giveups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
#pragma unroll
                for (int j = 0; j < TILES; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        if (wd[j][h] == kEmpty)
                            wd[j][h] = __hip_atomic_load(src + (j * kWave + lane) * 2 + h, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int j = 0; j < TILES; ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    __hip_atomic_store(src + (j * kWave + lane) * 2 + h, kEmpty, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                const u32x4 u = {(uint32_t)wd[j][0], (uint32_t)(wd[j][0] >> 32), (uint32_t)wd[j][1],
                                 (uint32_t)(wd[j][1] >> 32)};
                red[wave][j][lane] = __builtin_bit_cast(f32x4, u);
            }
        }
        __syncthreads();
        const int nw = min(WAVES, a.ksplit - s0);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = threadIdx.x + i * NTHR;
            if (e < ELEMS)
                for (int w = 0; w < nw; ++w)
                    v[i] += (s0 + w == rs) ? own[i] : red[w][e / kWave][e % kWave];
        }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * NTHR;
        if (e < ELEMS)
            store_out(e, v[i]);
    }
}

}  // namespace gdp
