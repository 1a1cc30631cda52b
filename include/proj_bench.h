/*
 * proj_bench.h - measurement kernels exported by the same library.
 *
 * The pages time every call with cold caches (guide ch. 1 "The problem, the
 * judge and the speed of light", §1.4: a buffer larger than the cache is read
 * before every replay) and compare each kernel with a hand-written pure-read
 * kernel of the same byte count (report "Muse Spark Open Kernel Challenge -
 * muse_bf16_proj", Method/tooling and Round 2: the measured HBM read floor).
 * On MI355X the weights also fit in the 256 MB Infinity Cache, so the flush
 * must read more than L2 plus that cache.
 *
 * All functions are launch-only on `stream` (hipStream_t, NULL = null stream)
 * and return a proj_status (proj.h).
 */
#ifndef PROJ_BENCH_H
#define PROJ_BENCH_H

#include <stddef.h>

#include "proj.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * proj_bench_flush - read `bytes` of device memory at `buf` (16-byte aligned,
 * bytes a multiple of 16). `sink` (device, at least 4096 uint32) receives a
 * word only when a data-dependent test on the values read succeeds, which
 * keeps every read live without a reduction. mode 0: non-temporal loads;
 * mode 1: plain loads (allocate in every cache level like the GEMV kernels'
 * weight stream). Used with a buffer of 1 GiB or more to evict L2 and the
 * Infinity Cache; other modes return PROJ_ERR_UNSUPPORTED.
 */
int proj_bench_flush(const void *buf, size_t bytes, void *sink, int mode, void *stream);

/*
 * proj_bench_read_floor - pure streaming read of `bytes` at `buf` (16-byte
 * aligned, bytes a multiple of 16) with the access pattern of the GEMV weight
 * stream: 16 bytes per lane, each wave reading its own contiguous run 1 KB
 * per load, `unroll` loads in flight per lane (1, 2, 4 or 8). `grid`
 * workgroups (0 = 1024) of `waves` wavefronts (0 = 8, at most 16) each read
 * a contiguous share; mode 0 non-temporal loads, mode 1 plain loads. `sink`
 * (device, at least `grid` uint32 words) is written as for proj_bench_flush.
 * ev_start/ev_stop: NULL, or events from proj_bench_event_create that then
 * bracket exactly this kernel's execution.
 */
int proj_bench_read_floor(const void *buf, size_t bytes, void *sink, void *stream,
                          int grid, int waves, int unroll, int mode, void *ev_start, void *ev_stop);

/*
 * proj_bench_stamp - one single-wave kernel that writes the GPU's
 * constant-rate wall clock (64-bit, ticking at proj_bench_wallclock_khz) to
 * ((uint64_t *)buf)[idx] (buf device, 8-byte aligned). Captured into a
 * graph before and after a load's kernels, two stamps give the span of
 * those kernels on the GPU (the gaps between them included), a replay's
 * time without the host launch path (guide ch. 1 §1.4 times graph
 * replays; the report's round 3 found the gaps between kernels worth a
 * microsecond each).
 */
int proj_bench_stamp(void *buf, int idx, void *stream);

/* proj_bench_wallclock_khz - tick rate of the proj_bench_stamp clock, in kHz. */
int proj_bench_wallclock_khz(int *khz);

/*
 * proj_run_timed - proj_run (cfg == NULL) or proj_run_config (cfg != NULL)
 * launched so that the two events, created by proj_bench_event_create, are
 * stamped at the start and the end of the kernel's own execution on the
 * GPU (hipExtLaunchKernel). This is the timing the bench reports as kernel
 * duration; it excludes the host/graph launch path. Not for graph capture.
 */
int proj_run_timed(int layer, const void *x, int m, void *out, void *stream,
                   const proj_config *cfg, void *ev_start, void *ev_stop);

/* Timing events (hipEvent_t) for proj_run_timed / proj_bench_read_floor. */
int proj_bench_event_create(void **ev);
int proj_bench_event_destroy(void *ev);
/* Waits for `stop` and writes the elapsed milliseconds between the events. */
int proj_bench_event_elapsed(void *start, void *stop, float *ms);

/*
 * proj_bench_copy - copy `bytes` (multiple of 16, both pointers 16-byte
 * aligned, no overlap) from `src` to `dst` with 16-byte loads and stores. A
 * kernel whose HBM read and write volumes are known exactly: hardware byte
 * counters read on it give the scale for the counters read on the GEMV
 * kernels.
 */
int proj_bench_copy(const void *src, void *dst, size_t bytes, void *stream);

/* proj_bench_empty - one empty kernel (measures launch/graph-node cost). */
int proj_bench_empty(void *stream);

/*
 * proj_bench_mfma_layout - one v_mfma_f32_16x16x32_bf16 with operands placed
 * at the lane positions the GEMV kernels assume: A is 16 x 32 row-major BF16
 * (A[i][k]), B is 32 x 16 row-major BF16 (B[k][j]), both device; the kernel
 * writes C = A B as 16 x 16 row-major FP32 (device) from the accumulator
 * lanes the kernels read results from. A test that feeds small integers and
 * compares with an exact product confirms the layout. One wave, no other
 * memory touched.
 */
int proj_bench_mfma_layout(const void *A, const void *B, void *C, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PROJ_BENCH_H */
