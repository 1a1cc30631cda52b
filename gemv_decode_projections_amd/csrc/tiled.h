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
//   * Activations (L2-resident) are loaded cooperatively, D k-steps ahead,
//     with quad-contiguous reads (each lane quad reads one token's 64-byte row
//     segment, the four k-groups rotated per token), then written to a 4-slot
//     LDS ring two k-steps ahead. The rotation makes both the 1 KB contiguous
//     LDS writes and the MFMA-layout reads (lane l: token l%16, k =
//     8*(l/16)+0..7) free of bank conflicts. Each k-step's B fragments are read
//     from LDS during the previous k-step's MFMAs. One barrier per k-step.
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

template <int RBW, int BNB, int WAVES, int D, bool F32W>
__global__ __launch_bounds__(WAVES * kWave) void tiled_kernel(TiledArgs a)
{
    constexpr int NTHR = WAVES * kWave;
    constexpr int AW = F32W ? 2 : 1;                  // 1 KB units per weight fragment
    constexpr int BMB = WAVES * RBW;                  // row blocks per tile
    static_assert(D >= 2 && (D & (D - 1)) == 0, "prefetch distance: power of two");
    static_assert((BNB * kWave) % NTHR == 0, "activation fragments must split over threads");
    constexpr int XPT = BNB * kWave / NTHR;           // activation units per thread per k-step

    __shared__ u32x4 xl[4][BNB * kWave];
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
    const int step0 = ks * steps;
    const int tok0 = tt * BNB * 16;
    const int rbw0 = rt * BMB + wave * RBW;          // first row block of this wave

    const u32x4 *wbase = reinterpret_cast<const u32x4 *>(a.wp);

    // Activation load plan for this thread (XPT units per k-step). Rows past
    // the last token read a zero row instead of being masked afterwards: a
    // select on loaded data gets hoisted next to the loads and forces waits.
    const uint16_t *xsrc[XPT];
    int xdst[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int u = i * NTHR + tid;
        const int blk = u / kWave;
        const int s = u % kWave;
        const int q = s / 4;                          // token within the 16-token block
        const int g = ((s % 4) - q / 4) & 3;          // rotated k-group
        const int tok = tok0 + blk * 16 + q;
        xsrc[i] = (tok < a.m ? a.x + (size_t)tok * a.K : a.zrow) + 8 * g;
        xdst[i] = u;                                  // LDS unit (fragment blk, slot s)
    }
    // LDS slot that holds (token l%16, k-group l/16) of a fragment for this lane.
    const int bslot = 4 * (lane % 16) + (((lane / 16) + (lane % 16) / 4) & 3);

    u32x4 wr[D][RBW][AW];
    u32x4 xr[D][XPT];
    u32x4 br[2][BNB];
    f32x4 acc[RBW][BNB];
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_w = [&](int slot, int j) {
        const int st = step0 + (j < steps ? j : steps - 1);
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
            const u32x4 *f = wbase + ((size_t)(rbw0 + r) * KS + st) * (AW * kWave) + lane;
#pragma unroll
            for (int h = 0; h < AW; ++h)
                wr[slot][r][h] = f[h * kWave];
        }
    };
    auto load_x = [&](int slot, int j) {
        const int st = step0 + (j < steps ? j : steps - 1);
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            xr[slot][i] = *reinterpret_cast<const u32x4 *>(xsrc[i] + (size_t)st * kStepK);
    };
    auto store_x = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            xl[buf][xdst[i]] = xr[slot][i];
    };
    auto read_b = [&](int reg, int buf) {
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            br[reg][t] = xl[buf][t * kWave + bslot];
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

    // Pipeline (4 LDS slots, D register slots, two B-fragment register sets):
    //   iteration j reads k-step j+1's fragments from LDS into br[(j+1)%2],
    //   multiplies k-step j (wr[j%D], br[j%2]), writes k-step j+2's
    //   activations from xr[(j+2)%D] to LDS slot (j+2)%4, refills wr[j%D] with
    //   k-step j+D and xr[(j+2)%D] with k-step j+D+2, then one barrier.
    // The LDS reads for the next k-step overlap this k-step's MFMAs; the
    // barrier publishes slot (j+2)%4 for iteration j+1 and retires the reads of
    // the slot that iteration j+2 overwrites (last read at iteration j-3).
    // The prologue leaves the loads in flight in the order the loop does.
    load_x(0, 0);
    load_x(1, 1);
    store_x(0, 0);
    store_x(1, 1);
#pragma unroll
    for (int j = 0; j < D; ++j) {
        load_w(j, j);
        load_x((j + 2) % D, j + 2);
    }
    __syncthreads();
    read_b(0, 0);

    for (int j0 = 0; j0 < steps; j0 += D) {
#pragma unroll
        for (int jj = 0; jj < D; ++jj) {
            const int j = j0 + jj;
            read_b((jj + 1) & 1, (jj + 1) & 3);
            compute(jj, jj & 1);
            store_x((jj + 2) % D, (jj + 2) & 3);
            load_w(jj, j + D);
            load_x((jj + 2) % D, j + D + 2);
            __syncthreads();
        }
    }

    // Epilogue. Accumulator (r, t) covers rows (rbw0 + r)*16 + 4*(lane/16) + 0..3
    // and token tok0 + t*16 + lane%16.
    auto store_out = [&](int r, int t, f32x4 v) {
        const int tk = tok0 + t * 16 + (lane % 16);
        if (tk >= a.m)
            return;
        const int row = (rbw0 + r) * kRowsPerBlock + 4 * (lane / 16);
        if constexpr (F32W) {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + (size_t)tk * a.n_eff + row) = v;
        } else {
            u32x2 p;
            p.x = bf16_rne_bits(v.x) | (bf16_rne_bits(v.y) << 16);
            p.y = bf16_rne_bits(v.z) | (bf16_rne_bits(v.w) << 16);
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + (size_t)tk * a.n_eff + row) = p;
        }
    };

    if (a.ksplit == 1) {
#pragma unroll
        for (int r = 0; r < RBW; ++r)
#pragma unroll
            for (int t = 0; t < BNB; ++t)
                store_out(r, t, acc[r][t]);
        return;
    }

    // Split-K: publish partials with agent-scope (write-through) stores, count
    // arrivals, and let the last workgroup of the tile sum the partials in split
    // order with agent-scope loads. Values move as 8-byte words, and the last
    // workgroup issues every load of one split before using any of them.
    constexpr int TILE_W = BMB * BNB * kWave * 2;     // 8-byte words per partial tile
    constexpr int NW = RBW * BNB * 2;                 // words per thread
    const int tile = rt * a.n_tt + tt;
    uint64_t *wsp = reinterpret_cast<uint64_t *>(a.ws) + (size_t)tile * a.ksplit * TILE_W;
    auto word_of = [&](int r, int t, int h) { return (((wave * RBW + r) * BNB + t) * kWave + lane) * 2 + h; };
    // Whole-vector bit casts only: a bit cast of a single vector element is
    // lowered by clang as a read of element 0.
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int t = 0; t < BNB; ++t) {
            const u32x4 u = __builtin_bit_cast(u32x4, acc[r][t]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint64_t w = (uint64_t)u[2 * h] | ((uint64_t)u[2 * h + 1] << 32);
                __hip_atomic_store(wsp + (size_t)ks * TILE_W + word_of(r, t, h), w, __ATOMIC_RELAXED,
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
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.ksplit; ++sp) {
        uint64_t part[NW];
        const uint64_t *src = wsp + (size_t)sp * TILE_W;
#pragma unroll
        for (int r = 0; r < RBW; ++r)
#pragma unroll
            for (int t = 0; t < BNB; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    part[(r * BNB + t) * 2 + h] =
                        __hip_atomic_load(src + word_of(r, t, h), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int r = 0; r < RBW; ++r)
#pragma unroll
            for (int t = 0; t < BNB; ++t) {
                const uint64_t w0 = part[(r * BNB + t) * 2];
                const uint64_t w1 = part[(r * BNB + t) * 2 + 1];
                const u32x4 u = {(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
                acc[r][t] += __builtin_bit_cast(f32x4, u);
            }
    }
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int t = 0; t < BNB; ++t)
            store_out(r, t, acc[r][t]);
    if (tid == 0)
        __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace gdp
