// Tiled MFMA kernel: out = x @ W^T when enough tokens share each weight byte
// that the work becomes a dense contraction (m >= 33; the pages' verify loads
// run m = 128 and 256, guide ch. 1 "The problem, the judge and the speed of
// light", §1.2, and only there do the big layers approach the math limit,
// §1.7).
//
// The report "Muse Spark Open Kernel Challenge - muse_bf16_proj" (round 4)
// traced its dense-layer losses to activations re-read by every row tile and
// to per-block ingest; both are the design constraints here, measured on
// MI355X: quad-contiguous L2 reads reach ~52 B/clk per compute unit, LDS reads
// ~142 B/clk, and one 16x16x32 MFMA takes 16 cycles per SIMD.
//
// gfx950 design:
//   * A workgroup owns WAVES*RBW 16-row blocks x BNB 16-token blocks and a K
//     range. Waves split the rows: wave w owns RBW row blocks and all BNB
//     token blocks, so no weight byte is loaded twice in a workgroup.
//   * Weights (the HBM stream) go straight into registers, each wave reading
//     its own 1 KB fragments (fragment-major packing, repack.h) D k-steps
//     ahead of use.
//   * Activations (L2-resident) are staged through a 4-slot LDS ring in
//     super-steps of S k-steps: consecutive lanes read one token's S*64
//     contiguous bytes, two super-steps ahead, and write them to the
//     positions the MFMA reads (lane l: token l%16, k = 8*(l/16)+0..7),
//     rotated per token and skewed per k-step so that both the writes and the
//     fragment reads are free of bank conflicts. Each k-step's B fragments are
//     read from LDS during the previous k-step's MFMAs. One barrier per
//     super-step: with one barrier per k-step the barriers alone cost about a
//     quarter of the kernel (measured by removing them).
//   * v_mfma_f32_16x16x32_bf16 with FP32 accumulation; FP32 router weights are
//     split exactly into three BF16 parts in registers (common.h).
//   * K may be split over KSPLIT workgroups per tile; the split index varies
//     fastest across workgroups, so one tile's workgroups sit on one XCD. The
//     last to arrive sums the partials in split order (deterministic) through
//     agent-scope (cache-coherent) accesses, as in skinny.h.
//   * Token rows past m read a library-owned zero row; their outputs are never
//     stored. Loads past the end of the K range are clamped to its last k-step
//     (cache hits, never consumed), which keeps the pipeline free of branches.
#pragma once

#include "common.h"

namespace gdp {

struct TiledArgs {
    const void *wp;          // packed weights
    const uint16_t *x;       // m x K BF16
    const uint16_t *zrow;    // K zero BF16 values (library-owned)
    void *out;               // m x n_eff
    float *ws;               // split-K partials
    uint32_t *counters;      // per-tile arrival counters, zero between launches
    int m;
    int K;
    int n_eff;
    int n_rt;                // row tiles
    int n_tt;                // token tiles
    int ksplit;
    int xcd_remap;
};

template <int RBW, int BNB, int WAVES, int S, int D, bool F32W>
__global__ __launch_bounds__(WAVES * kWave) void tiled_kernel(TiledArgs a)
{
    constexpr int NTHR = WAVES * kWave;
    constexpr int AW = F32W ? 2 : 1;                  // 1 KB units per weight fragment
    constexpr int BMB = WAVES * RBW;                  // row blocks per tile
    constexpr int PAD = S > 1 ? 4 : 0;                // units between k-step regions (bank skew)
    constexpr int REG = BNB * kWave + PAD;            // LDS units per k-step region
    constexpr int UNITS = S * BNB * kWave;            // 16-byte activation units per super-step
    constexpr int CPT = 4 * S;                        // 16-byte chunks per token per super-step
    static_assert(D >= S && D % S == 0 && (D & (D - 1)) == 0, "prefetch distance: power of two, whole super-steps");
    static_assert(S == 1 || S == 2 || S == 4, "k-steps per super-step");
    static_assert((D / S) % 2 == 0, "an even number of super-steps per unrolled pass (register ring of 2)");
    static_assert(UNITS % NTHR == 0, "activation units must split over threads");
    constexpr int XPT = UNITS / NTHR;                 // activation units per thread per super-step

    __shared__ u32x4 xl[4][S * REG];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;

    // Workgroup -> (split, token tile, row tile), split fastest.
    const int G = gridDim.x;
    int L = blockIdx.x;
    if (a.xcd_remap)
        L = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    const int ks = L % a.ksplit;
    const int rest = L / a.ksplit;
    const int tt = rest % a.n_tt;
    const int rt = rest / a.n_tt;

    const int KS = a.K / kStepK;
    const int steps = KS / a.ksplit;                  // k-steps of this workgroup (multiple of D)
    const int nss = steps / S;                        // super-steps
    const int step0 = ks * steps;
    const int tok0 = tt * BNB * 16;
    const int rbw0 = rt * BMB + wave * RBW;           // first row block of this wave

    const u32x4 *wbase = reinterpret_cast<const u32x4 *>(a.wp);

    // Activation load plan (XPT units per thread per super-step). Unit u reads
    // 16-byte chunk c = u % CPT of token u / CPT: consecutive lanes read one
    // token's S*64 contiguous bytes. Chunk c is k-step c/4, k-group c%4 of
    // the super-step; it lands in LDS at the MFMA-read position of that
    // k-group, rotated per token so that the fragment reads (lane l: token
    // l%16, k-group l/16) hit distinct banks; k-step regions are skewed by PAD
    // units so that the writes of one token's chunks do too. Rows past the
    // last token read a zero row instead of being masked afterwards: a select
    // on loaded data gets hoisted next to the loads and forces waits.
    const uint16_t *xsrc[XPT];
    int xdst[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int u = i * NTHR + tid;
        const int c = u % CPT;
        const int qt = u / CPT;                       // token within the tile
        const int blk = qt / 16, q = qt % 16;
        const int sub = c / 4, g = c % 4;
        const int tok = tok0 + qt;
        xsrc[i] = (tok < a.m ? a.x + (size_t)tok * a.K : a.zrow) + 8 * c;
        xdst[i] = sub * REG + blk * kWave + 4 * q + ((g + q / 4) & 3);
    }
    // LDS unit that holds (token l%16, k-group l/16) of a fragment for this lane.
    const int bslot = 4 * (lane % 16) + (((lane / 16) + (lane % 16) / 4) & 3);

    u32x4 wr[D][RBW][AW];
    u32x4 xr[2][XPT];
    u32x4 br[2][BNB];
    f32x4 acc[RBW][BNB];
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_w = [&](int slot, int j) {              // k-step j of this workgroup
        const int st = step0 + (j < steps ? j : steps - 1);
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
            const u32x4 *f = wbase + ((size_t)(rbw0 + r) * KS + st) * (AW * kWave) + lane;
#pragma unroll
            for (int h = 0; h < AW; ++h)
                wr[slot][r][h] = f[h * kWave];
        }
    };
    auto load_x = [&](int slot, int J) {              // super-step J
        const int st = step0 + (J < nss ? J : nss - 1) * S;
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            xr[slot][i] = *reinterpret_cast<const u32x4 *>(xsrc[i] + (size_t)st * kStepK);
    };
    auto store_x = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            xl[buf][xdst[i]] = xr[slot][i];
    };
    auto read_b = [&](int reg, int buf, int sub) {
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            br[reg][t] = xl[buf][sub * REG + t * kWave + bslot];
    };
    auto compute = [&](int slot, int reg) {
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
            if constexpr (F32W) {
                u32x4 hi, mid, lo;
                split3_f32(wr[slot][r][0], wr[slot][r][1], hi, mid, lo);
#pragma unroll
                for (int t = 0; t < BNB; ++t) {
                    acc[r][t] = mfma16x16x32(hi, br[reg][t], acc[r][t]);
                    acc[r][t] = mfma16x16x32(mid, br[reg][t], acc[r][t]);
                    acc[r][t] = mfma16x16x32(lo, br[reg][t], acc[r][t]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < BNB; ++t)
                    acc[r][t] = mfma16x16x32(wr[slot][r][0], br[reg][t], acc[r][t]);
            }
        }
    };

    // Pipeline. Weights: register ring of D k-steps, k-step j+D loaded while
    // k-step j is multiplied. Activations: super-step J+2 waits in registers
    // (loaded two iterations earlier) and is written to LDS slot (J+2)%4 at
    // iteration J; super-step J+4 is loaded in its place. Within iteration J,
    // each k-step's B fragments are read from LDS during the previous
    // k-step's MFMAs (across the super-step boundary too: slot (J+1)%4 was
    // published by the barrier of iteration J-1). One barrier per super-step
    // publishes slot (J+2)%4 and retires the reads of the slot iteration J+1
    // overwrites (last read during iteration J-2 and the prefetch at the end of
    // iteration J-3). The prologue leaves the loads in flight in the order the
    // loop does.
    load_x(0, 0);
    load_x(1, 1);
    store_x(0, 0);
    store_x(1, 1);
    load_x(0, 2);
    load_x(1, 3);
#pragma unroll
    for (int j = 0; j < D; ++j)
        load_w(j, j);
    __syncthreads();
    read_b(0, 0, 0);

    for (int j0 = 0; j0 < steps; j0 += D) {
#pragma unroll
        for (int jj = 0; jj < D; ++jj) {
            const int j = j0 + jj;
            const int J = j / S;                      // super-step of k-step j
            const int sub = jj % S;
            // k-step j+1: same super-step, or the first of the next one.
            if (sub + 1 < S)
                read_b((jj + 1) & 1, J & 3, sub + 1);
            else
                read_b((jj + 1) & 1, (J + 1) & 3, 0);
            compute(jj, jj & 1);
            load_w(jj, j + D);
            if (sub == S - 1) {
                const int xs = (jj / S) & 1;          // == J & 1: j0 / S is even
                store_x(xs, (J + 2) & 3);
                load_x(xs, J + 4);
                __syncthreads();
            }
        }
    }

    f32x4 fin[RBW][BNB];
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            fin[r][t] = acc[r][t];
    constexpr int RBH = RBW;
    const int rbf = rbw0;                             // first row block of this wave

    // Epilogue. fin (h, t) covers rows (rbf + h)*16 + 4*(lane/16) + 0..3 and
    // token tok0 + t*16 + lane%16. The tile is staged in LDS token-major (the
    // activation ring is free after the last barrier) and written out in
    // 16-byte chunks, consecutive lanes along one token's output row, so the
    // stores are whole cache lines instead of 8-byte pieces on 16 rows.
    constexpr int OB = F32W ? 4 : 2;                  // output bytes per element
    constexpr int ROWB = BMB * kRowsPerBlock * OB;    // bytes of one token's tile row
    constexpr int ROWP = ROWB + 16;                   // padded LDS row (bank skew)
    constexpr int CPR = ROWB / 16;                    // 16-byte chunks per token row
    static_assert(BNB * 16 * ROWP <= (int)sizeof(xl), "output tile must fit the activation ring");
    char *ot = reinterpret_cast<char *>(&xl[0][0]);
    auto store_tile = [&](f32x4 (&v)[RBH][BNB]) {
#pragma unroll
        for (int h = 0; h < RBH; ++h)
#pragma unroll
            for (int t = 0; t < BNB; ++t) {
                const int tl = t * 16 + (lane % 16);
                const int rl = (rbf - rt * BMB + h) * kRowsPerBlock + 4 * (lane / 16);
                char *d = ot + tl * ROWP + rl * OB;
                if constexpr (F32W) {
                    *reinterpret_cast<f32x4 *>(d) = v[h][t];
                } else {
                    u32x2 p;
                    p.x = pack_bf16x2(v[h][t].x, v[h][t].y);
                    p.y = pack_bf16x2(v[h][t].z, v[h][t].w);
                    *reinterpret_cast<u32x2 *>(d) = p;
                }
            }
        __syncthreads();
        char *obase = reinterpret_cast<char *>(a.out) + (size_t)rt * BMB * kRowsPerBlock * OB;
        for (int c = tid; c < BNB * 16 * CPR; c += NTHR) {
            const int tl = c / CPR, ck = c % CPR;
            const int tk = tok0 + tl;
            if (tk < a.m)
                *reinterpret_cast<u32x4 *>(obase + (size_t)tk * a.n_eff * OB + ck * 16) =
                    *reinterpret_cast<const u32x4 *>(ot + tl * ROWP + ck * 16);
        }
    };

    if (a.ksplit == 1) {
        store_tile(fin);
        return;
    }

    // Split-K over workgroups: publish partials with agent-scope (write-through,
    // visible to every XCD) 8-byte stores, wait until they are complete, count
    // the arrival, and let the last workgroup of the tile gather the partials
    // CH splits at a time with every load in flight, sum all splits in split
    // order (deterministic), store the output and reset the counter for the
    // next launch. (A variant where the last to arrive skips its own publish and
    // polls a second counter for the others measured slower: the poll round
    // trip costs more than the publish it saves.)
    constexpr int TILE_W = BMB * BNB * kWave * 2;     // 8-byte words per partial tile
    constexpr int NW = RBH * BNB * 2;                 // words per thread
    constexpr int CH = 4;                             // splits gathered per round
    const int tile = rt * a.n_tt + tt;
    uint64_t *wsp = reinterpret_cast<uint64_t *>(a.ws) + (size_t)tile * a.ksplit * TILE_W;
    auto word_of = [&](int h, int t, int w) { return (((wave * RBH + h) * BNB + t) * kWave + lane) * 2 + w; };
    // Whole-vector bit casts only: a bit cast of a single vector element is
    // lowered by clang as a read of element 0.
#pragma unroll
    for (int h = 0; h < RBH; ++h)
#pragma unroll
        for (int t = 0; t < BNB; ++t) {
            const u32x4 u = __builtin_bit_cast(u32x4, fin[h][t]);
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const uint64_t word = (uint64_t)u[2 * w] | ((uint64_t)u[2 * w + 1] << 32);
                __hip_atomic_store(wsp + (size_t)ks * TILE_W + word_of(h, t, w), word, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        uint32_t prev = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(a.ksplit - 1));
    }
    __syncthreads();
    if (!s_last)
        return;
    f32x4 sum[RBH][BNB];
#pragma unroll
    for (int h = 0; h < RBH; ++h)
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            sum[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < a.ksplit; c0 += CH) {
        uint64_t part[CH][NW];
#pragma unroll
        for (int ci = 0; ci < CH; ++ci) {
            // Splits past the end re-read the last one (valid memory, never summed).
            const int sp = min(c0 + ci, a.ksplit - 1);
            const uint64_t *src = wsp + (size_t)sp * TILE_W;
#pragma unroll
            for (int h = 0; h < RBH; ++h)
#pragma unroll
                for (int t = 0; t < BNB; ++t)
#pragma unroll
                    for (int w = 0; w < 2; ++w)
                        part[ci][(h * BNB + t) * 2 + w] =
                            __hip_atomic_load(src + word_of(h, t, w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int ci = 0; ci < CH; ++ci) {
            const int sp = c0 + ci;
            if (sp >= a.ksplit)
                break;
#pragma unroll
            for (int h = 0; h < RBH; ++h)
#pragma unroll
                for (int t = 0; t < BNB; ++t) {
                    if (sp == ks) {
                        sum[h][t] += fin[h][t];          // same bits as the published copy
                    } else {
                        const uint64_t w0 = part[ci][(h * BNB + t) * 2];
                        const uint64_t w1 = part[ci][(h * BNB + t) * 2 + 1];
                        const u32x4 u = {(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
                        sum[h][t] += __builtin_bit_cast(f32x4, u);
                    }
                }
        }
    }
    store_tile(sum);
    if (tid == 0)
        __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace gdp
