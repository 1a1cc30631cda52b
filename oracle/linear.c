/*
 * CPU oracle for the bias-free linear layer out = x @ W^T.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link or call this
 * file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 *
 * What it computes (guide ch. 1 "The problem, the judge and the speed of
 * light", §1.1): out[i, n] = sum over k of x[i, k] * W[n, k], x being m x K
 * BF16, W being N x K (BF16, or FP32 for the router), and the reference being
 * FP64 (§1.5). The notebook's "The mathematics of our projection" note states
 * the same definition as one dot product per (token row, output feature).
 *
 * Each output is an FP64 sum taken in ascending k. The decode of BF16 and FP32
 * to double is exact, and so is every product (8 x 24 significand bits fit in
 * 53), so the only rounding is the FP64 summation itself.
 *
 * Parallelism: OpenMP splits the (i, n) outputs between threads; each output
 * keeps its own ascending-k sum, so the thread count does not change a bit of
 * the result.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* x: m x K BF16 bits, W: n_rows x K BF16 bits (row-major), out: m x n_rows FP64. */
void oracle_linear_bf16w(const uint16_t *x, const uint16_t *W, int64_t m, int64_t n_rows,
                         int64_t K, double *out)
{
    int64_t total = m * n_rows;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < total; ++t) {
        int64_t i = t / n_rows;
        int64_t n = t % n_rows;
        const uint16_t *xr = x + i * K;
        const uint16_t *wr = W + n * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += bf16_to_double(xr[k]) * bf16_to_double(wr[k]);
        out[i * n_rows + n] = acc;
    }
}

/* Router form: x BF16 bits, W FP32 (row-major n_rows x K), out FP64. */
void oracle_linear_f32w(const uint16_t *x, const float *W, int64_t m, int64_t n_rows,
                        int64_t K, double *out)
{
    int64_t total = m * n_rows;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < total; ++t) {
        int64_t i = t / n_rows;
        int64_t n = t % n_rows;
        const uint16_t *xr = x + i * K;
        const float *wr = W + n * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += bf16_to_double(xr[k]) * (double)wr[k];
        out[i * n_rows + n] = acc;
    }
}

/*
 * Magnitude of each output's terms: mag[i][n] = sum over k of |x[i, k]| * |W[n, k]|,
 * in FP64, ascending k, from the same exact decode. An FP32 accumulation of the
 * terms in any order is off from the exact sum by at most a multiple of this
 * value (the standard error bound of a floating-point sum), so it scales the
 * per-element part of the acceptance check (notebook note "Numerical formats
 * and error": BF16 operands, FP32 accumulation, an order that is free).
 */
void oracle_magnitude_bf16w(const uint16_t *x, const uint16_t *W, int64_t m, int64_t n_rows,
                            int64_t K, double *mag)
{
    int64_t total = m * n_rows;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < total; ++t) {
        int64_t i = t / n_rows;
        int64_t n = t % n_rows;
        const uint16_t *xr = x + i * K;
        const uint16_t *wr = W + n * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += fabs(bf16_to_double(xr[k])) * fabs(bf16_to_double(wr[k]));
        mag[i * n_rows + n] = acc;
    }
}

/* Router form of oracle_magnitude_bf16w: FP32 weights. */
void oracle_magnitude_f32w(const uint16_t *x, const float *W, int64_t m, int64_t n_rows,
                           int64_t K, double *mag)
{
    int64_t total = m * n_rows;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < total; ++t) {
        int64_t i = t / n_rows;
        int64_t n = t % n_rows;
        const uint16_t *xr = x + i * K;
        const float *wr = W + n * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += fabs(bf16_to_double(xr[k])) * fabs((double)wr[k]);
        mag[i * n_rows + n] = acc;
    }
}

/* Threads a parallel region will use (reported next to CPU timings). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* Set the thread count for later calls (1 gives the single-thread timing). */
void oracle_set_threads(int n) { omp_set_num_threads(n); }
