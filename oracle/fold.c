/*
 * In-order reduction folds for the CPU oracle (test infrastructure only).
 *
 * Each function folds `cells` independent rows of `n` contiguous values,
 * row c occupying x[c*n .. c*n+n-1], walking every row in ascending order
 * from the reduce identity. This is the fold order of limn's reference loop
 * nest (limn README, "Reading the schedule": the reduce identity is stored
 * first and each value is folded into it with ACCUM; "Backends": the c device
 * threads only the output cells, so each cell is still folded start to
 * finish by one thread in the serial order). Threads split cells, never a
 * row, so a threaded run gives the same bits as a serial one.
 *
 * Accumulator widths follow limn README, "The op set" (dtype paragraph):
 * float32 running totals for float32/float16/bfloat16 data, float64 for
 * float64, and wrap-around integer arithmetic modulo 2^32 for the ints.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>

void fold_sum_f32(const float* x, int64_t cells, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const float* row = x + c * n;
        float acc = 0.0f;
        for (int64_t i = 0; i < n; ++i) acc = acc + row[i];
        out[c] = acc;
    }
}

/* float32 data with a float64 running total, rounded once to float32. */
void fold_sum_f32_wide(const float* x, int64_t cells, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const float* row = x + c * n;
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) acc = acc + (double)row[i];
        out[c] = (float)acc;
    }
}

/* float32 data with a float64 running total, returned unrounded. */
void fold_sum_f32_to_f64(const float* x, int64_t cells, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const float* row = x + c * n;
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) acc = acc + (double)row[i];
        out[c] = acc;
    }
}

void fold_sum_f64(const double* x, int64_t cells, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const double* row = x + c * n;
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) acc = acc + row[i];
        out[c] = acc;
    }
}

void fold_sum_i32(const int32_t* x, int64_t cells, int64_t n, int32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const int32_t* row = x + c * n;
        uint32_t acc = 0u;
        for (int64_t i = 0; i < n; ++i) acc = acc + (uint32_t)row[i];
        out[c] = (int32_t)acc;
    }
}

/* MAX: identity -inf; a NaN anywhere in the row makes the result NaN. */
void fold_max_f32(const float* x, int64_t cells, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const float* row = x + c * n;
        float acc = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            float v = row[i];
            if (isnan(acc)) break;
            /* -0 orders below +0, so the result does not depend on the order */
            if (isnan(v) || v > acc || (v == acc && signbit(acc) && !signbit(v))) acc = v;
        }
        out[c] = acc;
    }
}

void fold_max_f64(const double* x, int64_t cells, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const double* row = x + c * n;
        double acc = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double v = row[i];
            if (isnan(acc)) break;
            /* -0 orders below +0, so the result does not depend on the order */
            if (isnan(v) || v > acc || (v == acc && signbit(acc) && !signbit(v))) acc = v;
        }
        out[c] = acc;
    }
}

/* Integer MAX: identity is the smallest value of the storage width. */
void fold_max_i32(const int32_t* x, int64_t cells, int64_t n, int32_t ident, int32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cells; ++c) {
        const int32_t* row = x + c * n;
        int32_t acc = ident;
        for (int64_t i = 0; i < n; ++i) if (row[i] > acc) acc = row[i];
        out[c] = acc;
    }
}
