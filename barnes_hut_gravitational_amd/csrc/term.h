// The softened monopole term shared by the walk and the direct sum, as a
// sequence of correctly rounded float32 operations (the library is compiled
// without contraction): r2 = ((dx*dx + dy*dy) + dz*dz) + eps^2,
// inv = RN(1 / RN(sqrt(r2))), f = m * ((inv * inv) * inv), a += f * d
// (softening and force law of the orrery performance page, "Accuracy").
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace orr {

// RN(1 / RN(sqrt(x))) for x in [2^-96, FLT_MAX] without the range scaling and
// special-value handling of the general IEEE sequences, which this domain
// never needs (x >= eps^2 >= 2^-96). sqrt: the hardware estimate is within one
// ulp; the correctly rounded root is chosen among it and its two neighbours by
// the signs of the exact residuals x - s'*s (fma). Reciprocal: the hardware
// estimate refined by one Newton step y += y * (1 - s*y) in fma, which is
// correctly rounded for every s = sqrt(x) of this domain. x = +inf (only from
// coordinate differences beyond float range) is clamped to FLT_MAX: its
// inverse cube then underflows to 0, as 1/inf cubed does; kClamp = false
// leaves the clamp out where no r2 can overflow. Equality of the cube with the
// IEEE operations' cube for every float in [2^-96, +inf] is checked by
// orr_selftest_inv_sqrt.
template <bool kClamp = true>
__device__ __forceinline__ float inv_sqrt_rn(float x) {
    if (kClamp) x = fminf(x, 3.40282347e38f);
    float s = __builtin_amdgcn_sqrtf(x);
    const float sm = __uint_as_float(__float_as_uint(s) - 1u);
    const float sp = __uint_as_float(__float_as_uint(s) + 1u);
    const float rm = fmaf(-sm, s, x);
    const float rp = fmaf(-sp, s, x);
    s = (rm <= 0.0f) ? sm : s;
    s = (rp > 0.0f) ? sp : s;
    const float y = __builtin_amdgcn_rcpf(s);
    const float e = fmaf(-s, y, 1.0f);
    return fmaf(e, y, y);
}

// a += m * d * r2^(-3/2) with r2 = |d|^2 + eps^2 given, every step one
// correctly rounded float operation (the library is compiled without
// contraction). The entry points admit only eps with eps^2 >= 2^-96 (a finite
// inverse cube of eps needs far more), so every r2 lies in inv_sqrt_rn's
// domain. kInv: 1 = inv_sqrt_rn (the cube of the IEEE square root and
// division on that domain); 2 = the same without the overflow clamp.
enum { kInvFast = 1, kInvFastNoClamp = 2 };

template <int kInv>
__device__ __forceinline__ void add_term_r2(float m, float dx, float dy, float dz, float r2, float &ax, float &ay,
                                            float &az) {
    const float inv = inv_sqrt_rn<kInv == kInvFast>(r2);
    const float f = m * ((inv * inv) * inv);
    ax += f * dx;
    ay += f * dy;
    az += f * dz;
}

// The same with r2 = ((dx*dx + dy*dy) + dz*dz) + eps2.
template <int kInv>
__device__ __forceinline__ void add_term(float m, float dx, float dy, float dz, float eps2, float &ax, float &ay,
                                         float &az) {
    add_term_r2<kInv>(m, dx, dy, dz, ((dx * dx + dy * dy) + dz * dz) + eps2, ax, ay, az);
}

// The term's product f * d alone (same operations as add_term_r2 before its
// three additions), for terms whose accumulation happens in another lane.
template <int kInv>
__device__ __forceinline__ float4 term_product(float m, float dx, float dy, float dz, float eps2) {
    const float r2 = ((dx * dx + dy * dy) + dz * dz) + eps2;
    const float inv = inv_sqrt_rn<kInv == kInvFast>(r2);
    const float f = m * ((inv * inv) * inv);
    return make_float4(f * dx, f * dy, f * dz, 0.0f);
}

}  // namespace orr
