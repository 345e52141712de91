/*
 * Alternative arithmetic for the softened monopole term, for the accuracy
 * experiment in tests/test_term_accuracy.py (test code only). Each function
 * sums n terms (m, dx, dy, dz) in the given order into a[3], the way one
 * target's walk adds them:
 *   sum_exact: the library's and the oracle's sequence, every step one
 *     correctly rounded float operation, inv = RN(1 / RN(sqrt(r2)));
 *   sum_rsqrt: the same with inv = RN(1 / sqrt(r2)) (one rounding, as a
 *     correctly rounded reciprocal square root instruction would give);
 *   sum_rsqrt_fma: that, plus fused multiply-adds in r2 and in a += f d;
 *   sum_exact_fma_acc: the exact sequence with only a += f d fused.
 * RN(1 / sqrt(r2)) is taken as the double reciprocal square root rounded to
 * float (double rounding is off only when the double lies within 2^-53 of a
 * float midpoint). Compiled with -ffp-contract=off; fmaf is the C library's
 * correctly rounded fused multiply-add.
 */
#include <math.h>
#include <stdint.h>

void sum_exact(const float *t, int64_t n, float eps2, float a[3]) {
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    for (int64_t k = 0; k < n; k++) {
        const float m = t[4 * k], dx = t[4 * k + 1], dy = t[4 * k + 2], dz = t[4 * k + 3];
        const float r2 = ((dx * dx + dy * dy) + dz * dz) + eps2;
        const float inv = 1.0f / sqrtf(r2);
        const float f = m * ((inv * inv) * inv);
        ax += f * dx;
        ay += f * dy;
        az += f * dz;
    }
    a[0] = ax, a[1] = ay, a[2] = az;
}

void sum_rsqrt(const float *t, int64_t n, float eps2, float a[3]) {
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    for (int64_t k = 0; k < n; k++) {
        const float m = t[4 * k], dx = t[4 * k + 1], dy = t[4 * k + 2], dz = t[4 * k + 3];
        const float r2 = ((dx * dx + dy * dy) + dz * dz) + eps2;
        const float inv = (float)(1.0 / sqrt((double)r2));
        const float f = m * ((inv * inv) * inv);
        ax += f * dx;
        ay += f * dy;
        az += f * dz;
    }
    a[0] = ax, a[1] = ay, a[2] = az;
}

void sum_rsqrt_fma(const float *t, int64_t n, float eps2, float a[3]) {
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    for (int64_t k = 0; k < n; k++) {
        const float m = t[4 * k], dx = t[4 * k + 1], dy = t[4 * k + 2], dz = t[4 * k + 3];
        const float r2 = fmaf(dz, dz, fmaf(dy, dy, fmaf(dx, dx, eps2)));
        const float inv = (float)(1.0 / sqrt((double)r2));
        const float f = m * ((inv * inv) * inv);
        ax = fmaf(f, dx, ax);
        ay = fmaf(f, dy, ay);
        az = fmaf(f, dz, az);
    }
    a[0] = ax, a[1] = ay, a[2] = az;
}

void sum_exact_fma_acc(const float *t, int64_t n, float eps2, float a[3]) {
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    for (int64_t k = 0; k < n; k++) {
        const float m = t[4 * k], dx = t[4 * k + 1], dy = t[4 * k + 2], dz = t[4 * k + 3];
        const float r2 = ((dx * dx + dy * dy) + dz * dz) + eps2;
        const float inv = 1.0f / sqrtf(r2);
        const float f = m * ((inv * inv) * inv);
        ax = fmaf(f, dx, ax);
        ay = fmaf(f, dy, ay);
        az = fmaf(f, dz, az);
    }
    a[0] = ax, a[1] = ay, a[2] = az;
}
