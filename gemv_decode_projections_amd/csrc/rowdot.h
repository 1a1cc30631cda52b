// Row-dot kernel: out = x @ W^T for up to 8 tokens on layers with few rows.
//
// The small layers of the decode loads (the FP32 router, 256 rows, and the
// 1024-row slice of the unpooler, guide ch. 1 "The problem, the judge and the
// speed of light", §1.1) hold only 16 or 64 blocks of 16 rows. A 16-row MFMA
// tile per workgroup leaves most of the 256 compute units idle, and splitting
// K over workgroups adds a publish / count / gather round trip through
// memory (about 2 us measured). Here a workgroup owns R whole rows instead, so
// the grid has hundreds of workgroups and no cross-workgroup reduction.
//
// gfx950 design:
//   * Weights are a row-major copy kept beside the fragment-major one; each
//     wave reads 1 KB contiguous per 16-byte-per-lane load and every load of
//     the workgroup is issued before the first multiply.
//   * Thread t covers k = i*2048 + 8t + 0..7 (one 16-byte activation load per
//     token, one or two 16-byte weight loads per row) for every row and
//     token of the workgroup, with one FP32 fused multiply-add per product
//     (BF16 activations are exact in FP32, so an FP32 weight enters the
//     product at full precision).
//   * The 64 lanes reduce their R*M partial sums with a halving butterfly
//     (each step keeps half of the values and adds the partner lane's copy),
//     then the four waves' results are summed through LDS in wave order. The
//     order of every addition is fixed, so results are bit-reproducible.
//   * Token rows past m read row m-1 and are never stored.
#pragma once

#include <type_traits>

#include "common.h"

namespace gdp {

constexpr int kRowWaves = 4;
constexpr int kRowThreads = kRowWaves * kWave;

struct RowArgs {
    const void *w;          // row-major weights, n_eff x K (FP32 or BF16)
    const uint16_t *x;      // m x K BF16
    void *out;              // m x n_eff (FP32 or BF16)
    int m;
    int K;
    int n_eff;
};

__device__ __forceinline__ float f32_of_bits(uint32_t u) { return __builtin_bit_cast(float, u); }

template <int M, int R, int KIT, bool F32W>
__global__ __launch_bounds__(kRowThreads) void rowdot_kernel(RowArgs a)
{
    constexpr int E = 8;                              // consecutive k per thread and chunk
    constexpr int KW = kRowThreads * E;               // k covered by one pass of the workgroup
    constexpr int AW = F32W ? 2 : 1;                  // 16-byte weight loads per chunk
    constexpr int V = R * M;                          // partial sums per thread
    static_assert(V <= kWave && (V & (V - 1)) == 0, "R*M: a power of two up to 64");

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int row0 = blockIdx.x * R;

    // Every load of the workgroup is issued before the first multiply; the
    // scheduling barrier keeps the compiler from interleaving them with the
    // arithmetic (which would serialize memory round trips).
    u32x4 wv[R][KIT][AW];
    u32x4 xv[M][KIT];
    const u32x4 *wbase = static_cast<const u32x4 *>(a.w);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < KIT; ++i)
#pragma unroll
            for (int h = 0; h < AW; ++h)
                wv[r][i][h] = wbase[((size_t)(row0 + r) * a.K + i * KW + tid * E) / (8 / AW) + h];
#pragma unroll
    for (int t = 0; t < M; ++t) {
        const int tok = t < a.m ? t : a.m - 1;
#pragma unroll
        for (int i = 0; i < KIT; ++i)
            xv[t][i] = *reinterpret_cast<const u32x4 *>(a.x + (size_t)tok * a.K + i * KW + tid * E);
    }
    __builtin_amdgcn_sched_barrier(0);

    // A vector value rather than an array: a lane-dependent choice between two
    // array elements would be turned into a variable index (a select chain).
    typedef float AccV __attribute__((ext_vector_type(V)));
    AccV acc;
#pragma unroll
    for (int v = 0; v < V; ++v)
        acc[v] = 0.f;
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
        float xf[M][E];
#pragma unroll
        for (int t = 0; t < M; ++t)
#pragma unroll
            for (int j = 0; j < E / 2; ++j) {
                const uint32_t q = xv[t][i][j];
                xf[t][2 * j] = f32_of_bits(q << 16);
                xf[t][2 * j + 1] = f32_of_bits(q & 0xffff0000u);
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float wf[E];
#pragma unroll
            for (int h = 0; h < AW; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t q = wv[r][i][h][j];
                    if constexpr (F32W) {
                        wf[4 * h + j] = f32_of_bits(q);
                    } else {
                        wf[2 * j] = f32_of_bits(q << 16);
                        wf[2 * j + 1] = f32_of_bits(q & 0xffff0000u);
                    }
                }
#pragma unroll
            for (int t = 0; t < M; ++t)
#pragma unroll
                for (int j = 0; j < E; ++j)
                    acc[r * M + t] = __builtin_fmaf(xf[t][j], wf[j], acc[r * M + t]);
        }
    }

    // Halving butterfly over the wave: at offset o a lane keeps the lower half
    // of its values if (lane & o) == 0, else the upper half, and adds the
    // partner's copy of the half it keeps. After log2(V) halvings lane l holds
    // value l >> (6 - log2 V); the remaining offsets are full butterflies.
    constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4 : V == 32 ? 5 : 6;
    constexpr int SH = 6 - LOGV;
    // Counted loops with constant bounds so that every index is a constant
    // after unrolling (a variable index into acc[] becomes a select chain).
#pragma unroll
    for (int lvl = 0; lvl < LOGV; ++lvl) {
        const int o = (kWave / 2) >> lvl;
        const int half = V >> (lvl + 1);
        const bool upper = (lane & o) != 0;
#pragma unroll
        for (int p = 0; p < half; ++p) {
            const float send = upper ? acc[p] : acc[half + p];
            const float keep = upper ? acc[half + p] : acc[p];
            acc[p] = keep + __shfl_xor(send, o);
        }
    }
#pragma unroll
    for (int lvl = LOGV; lvl < 6; ++lvl)
        acc[0] += __shfl_xor(acc[0], (kWave / 2) >> lvl);
    __shared__ float red[kRowWaves][V];
    if ((lane & ((1 << SH) - 1)) == 0)
        red[wave][lane >> SH] = acc[0];
    __syncthreads();
    if (tid < V) {
        float s = red[0][tid];
#pragma unroll
        for (int w = 1; w < kRowWaves; ++w)
            s += red[w][tid];
        const int r = tid / M, t = tid % M;
        if (t < a.m) {
            const size_t o = (size_t)t * a.n_eff + row0 + r;
            if constexpr (F32W)
                static_cast<float *>(a.out)[o] = s;
            else
                static_cast<uint16_t *>(a.out)[o] = (uint16_t)pack_bf16x2(s, 0.f);
        }
    }
}

}  // namespace gdp
