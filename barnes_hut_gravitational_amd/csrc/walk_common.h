// Pieces shared by the walk kernels: block size, the XCD-contiguous block
// order, the output writer (scatter to the caller's order through perm) and
// the bound under which no r2 can overflow.
#pragma once

#include <cmath>

#include "orr_internal.h"

#ifndef ORR_WALK_BLOCK
#define ORR_WALK_BLOCK 256
#endif

namespace orr {

constexpr uint32_t kWalkBlock = ORR_WALK_BLOCK;  // threads per block (multiple of 64)

// Blocks are handed to the 8 XCDs round-robin; the independent walk gives
// each XCD a contiguous run of target blocks, so that its L2 holds one region
// of the tree for the per-lane node loads.
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t nblocks) {
    const uint32_t x = b & 7u, q = nblocks >> 3, r = nblocks & 7u;
    return x * q + min(x, r) + (b >> 3);
}

struct WalkOut {
    float *acc;
    uint32_t *visits_own, *visits_stepped, *n_pp, *n_pc;
};

__device__ __forceinline__ void write_out(const WalkOut &o, uint32_t dst, float ax, float ay, float az,
                                          uint32_t vown, uint32_t vstep, uint32_t pp, uint32_t pc) {
    if (o.acc) {
        o.acc[3ull * dst] = ax;
        o.acc[3ull * dst + 1] = ay;
        o.acc[3ull * dst + 2] = az;
    }
    if (o.visits_own) o.visits_own[dst] = vown;
    if (o.visits_stepped) o.visits_stepped[dst] = vstep;
    if (o.n_pp) o.n_pp[dst] = pp;
    if (o.n_pc) o.n_pc[dst] = pc;
}

// r2 <= 3 (side (1 + 2^-20))^2 + eps2 for every pair inside the root cube,
// coms included; below this bound no r2 can overflow float.
__device__ __forceinline__ bool r2_cannot_overflow(const DevParams *prm, float eps2) {
    const double s = (double)prm->side * (1.0 + 0x1p-20);
    return 3.0 * s * s + (double)eps2 < 1e38;
}

// Every node's s^2 is RN(side^2) 2^-2l for its level l <= 21 (s = side 2^-l
// exactly); s^2 2^e stays a normal float for all of them when the exponent
// field of RN(side^2) is at least 1 + 2 * 21 and at most 254 - e.
__device__ __forceinline__ bool pow2_scale_ok(const DevParams *prm, uint32_t e) {
    if (e > 126u) return false;
    const float L2 = prm->side * prm->side;
    const uint32_t ex = (__float_as_uint(L2) >> 23) & 0xffu;
    return ex >= 1u + 2u * (uint32_t)kMaxLevel && ex + e <= 254u;
}

// e with theta2 = 2^-e exactly, 0 <= e <= 126; kNotPow2 otherwise.
constexpr uint32_t kNotPow2 = 0xffffffffu;
inline uint32_t theta2_pow2_exp(float theta2) {
    if (!(theta2 > 0.0f && theta2 <= 1.0f)) return kNotPow2;
    int ex = 0;
    const float m = std::frexp(theta2, &ex);  // theta2 = m 2^ex, m in [0.5, 1)
    if (m != 0.5f || 1 - ex > 126) return kNotPow2;
    return (uint32_t)(1 - ex);
}

}  // namespace orr
