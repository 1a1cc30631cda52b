// Measurement kernels: cache flush, pure-read floor, empty kernel, MFMA
// lane-layout check. Declarations and contracts are in proj_bench.h.
#include <hip/hip_ext.h>

#include "../../include/proj.h"
#include "../../include/proj_bench.h"
#include "common.h"

namespace gdp {
namespace {

constexpr uint32_t kSinkMagic = 0x9e3779b9u;   // data-dependent store keeps reads live

// One 16-byte load: non-temporal (NT) or plain (cached like the GEMV
// kernels' weight stream).
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4 *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void flush_kernel(const u32x4 *__restrict__ buf, size_t units,
                                                     uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < units; i += 4 * stride) {
        u32x4 a = load16<NT>(buf + i);
        u32x4 b = load16<NT>(buf + i + stride);
        u32x4 c = load16<NT>(buf + i + 2 * stride);
        u32x4 d = load16<NT>(buf + i + 3 * stride);
        acc ^= a.x ^ b.y ^ c.z ^ d.w;
    }
    for (; i < units; i += stride) {
        u32x4 a = load16<NT>(buf + i);
        acc ^= a.x;
    }
    if (acc == kSinkMagic)
        sink[blockIdx.x] = acc;
}

template <int UNROLL, bool NT>
__global__ __launch_bounds__(1024) void read_floor_kernel(const u32x4 *__restrict__ buf, size_t units,
                                                           size_t per_wg, size_t per_wave,
                                                           uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const size_t wg_begin = (size_t)blockIdx.x * per_wg;
    const size_t wg_end = wg_begin + per_wg < units ? wg_begin + per_wg : units;
    size_t begin = wg_begin + (size_t)wave * per_wave;
    size_t end = begin + per_wave < wg_end ? begin + per_wave : wg_end;
    uint32_t acc = 0;
    size_t i = begin + lane;
    for (; i + (UNROLL - 1) * kWave < end; i += UNROLL * kWave) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = load16<NT>(buf + i + u * kWave);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            acc ^= v[u].x ^ v[u].w;
    }
    for (; i < end; i += kWave)
        acc ^= load16<NT>(buf + i).y;
    if (acc == kSinkMagic)
        sink[blockIdx.x] = acc;
}

// One lane writes the GPU's constant-rate wall clock (s_memrealtime) to
// out[idx]. Placed before and after a load's kernels inside a graph, two
// stamps give the span of those kernels on the GPU, gaps between them
// included, without the host's launch path.
__global__ __launch_bounds__(64) void stamp_kernel(uint64_t *__restrict__ out, int idx)
{
    const uint64_t t = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0)
        out[idx] = t;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                    size_t units)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < units; i += stride)
        dst[i] = src[i];
}

__global__ void empty_kernel() {}

// One wave: operands placed as the GEMV kernels place them (common.h).
__global__ __launch_bounds__(64) void mfma_layout_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B,
                                                         float *__restrict__ C)
{
    const int l = threadIdx.x;
    uint16_t a[8], b[8];
    for (int e = 0; e < 8; ++e) {
        a[e] = A[(l % 16) * 32 + 8 * (l / 16) + e];     // A[row l%16][k]
        b[e] = B[(8 * (l / 16) + e) * 16 + (l % 16)];   // B[k][col l%16]
    }
    u32x4 av, bv;
    for (int j = 0; j < 4; ++j) {
        av[j] = (uint32_t)a[2 * j] | ((uint32_t)a[2 * j + 1] << 16);
        bv[j] = (uint32_t)b[2 * j] | ((uint32_t)b[2 * j + 1] << 16);
    }
    f32x4 c = mfma16x16x32(av, bv, f32x4{0.f, 0.f, 0.f, 0.f});
    for (int i = 0; i < 4; ++i)
        C[(4 * (l / 16) + i) * 16 + (l % 16)] = c[i];    // C[row][col l%16]
}

int hip_status(hipError_t e) { return e == hipSuccess ? PROJ_OK : PROJ_ERR_HIP; }

}  // namespace
}  // namespace gdp

using namespace gdp;

extern "C" {

int proj_bench_flush(const void *buf, size_t bytes, void *sink, int mode, void *stream)
{
    if (!buf || !sink)
        return PROJ_ERR_NULL;
    if (((uintptr_t)buf & 15u) || (bytes & 15u))
        return PROJ_ERR_ALIGN;
    if (mode != 0 && mode != 1)
        return PROJ_ERR_UNSUPPORTED;
    if (mode == 0)
        hipLaunchKernelGGL(flush_kernel<true>, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u32x4 *>(buf), bytes / 16, static_cast<uint32_t *>(sink));
    else
        hipLaunchKernelGGL(flush_kernel<false>, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u32x4 *>(buf), bytes / 16, static_cast<uint32_t *>(sink));
    return hip_status(hipGetLastError());
}

int proj_bench_read_floor(const void *buf, size_t bytes, void *sink, void *stream, int grid, int waves,
                          int unroll, int mode, void *ev_start, void *ev_stop)
{
    if (!buf || !sink)
        return PROJ_ERR_NULL;
    if (((uintptr_t)buf & 15u) || (bytes & 15u))
        return PROJ_ERR_ALIGN;
    if (grid <= 0)
        grid = 1024;
    if (waves <= 0)
        waves = 8;
    if (waves > 16 || (mode != 0 && mode != 1))
        return PROJ_ERR_UNSUPPORTED;
    const size_t units = bytes / 16;
    size_t per_wg = (units + grid - 1) / grid;
    size_t per_wave = (per_wg + waves - 1) / waves;
    per_wave = (per_wave + kWave - 1) / kWave * kWave;   // each wave starts 1 KB-aligned
    per_wg = per_wave * waves;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *b = static_cast<const u32x4 *>(buf);
    uint32_t *k = static_cast<uint32_t *>(sink);
    dim3 g(grid), blk(waves * kWave);
    const void *fn;
    switch (unroll * 2 + mode) {
    case 2: fn = reinterpret_cast<const void *>(&read_floor_kernel<1, true>); break;
    case 3: fn = reinterpret_cast<const void *>(&read_floor_kernel<1, false>); break;
    case 4: fn = reinterpret_cast<const void *>(&read_floor_kernel<2, true>); break;
    case 5: fn = reinterpret_cast<const void *>(&read_floor_kernel<2, false>); break;
    case 8: fn = reinterpret_cast<const void *>(&read_floor_kernel<4, true>); break;
    case 9: fn = reinterpret_cast<const void *>(&read_floor_kernel<4, false>); break;
    case 16: fn = reinterpret_cast<const void *>(&read_floor_kernel<8, true>); break;
    case 17: fn = reinterpret_cast<const void *>(&read_floor_kernel<8, false>); break;
    default: return PROJ_ERR_UNSUPPORTED;
    }
    void *params[] = {&b, const_cast<size_t *>(&units), &per_wg, &per_wave, &k};
    hipError_t e;
    if (ev_start || ev_stop)
        e = hipExtLaunchKernel(fn, g, blk, params, 0, s, static_cast<hipEvent_t>(ev_start),
                               static_cast<hipEvent_t>(ev_stop), 0);
    else
        e = hipLaunchKernel(fn, g, blk, params, 0, s);
    return hip_status(e);
}

int proj_bench_event_create(void **ev)
{
    if (!ev)
        return PROJ_ERR_NULL;
    hipEvent_t e = nullptr;
    hipError_t r = hipEventCreate(&e);
    *ev = e;
    return hip_status(r);
}

int proj_bench_event_destroy(void *ev)
{
    if (!ev)
        return PROJ_OK;
    return hip_status(hipEventDestroy(static_cast<hipEvent_t>(ev)));
}

int proj_bench_event_elapsed(void *start, void *stop, float *ms)
{
    if (!start || !stop || !ms)
        return PROJ_ERR_NULL;
    hipError_t r = hipEventSynchronize(static_cast<hipEvent_t>(stop));
    if (r != hipSuccess)
        return PROJ_ERR_HIP;
    return hip_status(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)));
}

int proj_bench_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (!src || !dst)
        return PROJ_ERR_NULL;
    if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || (bytes & 15u))
        return PROJ_ERR_ALIGN;
    hipLaunchKernelGGL(copy_kernel, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), bytes / 16);
    return hip_status(hipGetLastError());
}

int proj_bench_stamp(void *buf, int idx, void *stream)
{
    if (!buf)
        return PROJ_ERR_NULL;
    if (((uintptr_t)buf & 7u) || idx < 0)
        return PROJ_ERR_ALIGN;
    hipLaunchKernelGGL(stamp_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint64_t *>(buf), idx);
    return hip_status(hipGetLastError());
}

int proj_bench_wallclock_khz(int *khz)
{
    if (!khz)
        return PROJ_ERR_NULL;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
    return hip_status(e);
}

int proj_bench_empty(void *stream)
{
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return hip_status(hipGetLastError());
}

int proj_bench_mfma_layout(const void *A, const void *B, void *C, void *stream)
{
    if (!A || !B || !C)
        return PROJ_ERR_NULL;
    hipLaunchKernelGGL(mfma_layout_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(B),
                       static_cast<float *>(C));
    return hip_status(hipGetLastError());
}

}  // extern "C"
