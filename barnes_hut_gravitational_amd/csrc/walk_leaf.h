// The opened-leaf evaluation shared by the production-style walks (walk.hip,
// walk_width.hip): a leaf that some lanes of a wave open is read once for all
// of them, staged in the wave's LDS with one coalesced load, and, when few
// lanes open it, its terms are packed across the wave's lanes. Every opening
// lane adds its leaf's terms in particle order with the operations of term.h,
// as its own walk would.
#pragma once

#include "orr_internal.h"
#include "term.h"
#include "walk_common.h"

#ifndef ORR_PACK_KMAX
#define ORR_PACK_KMAX 64  // pack leaf rows when at most this many lanes open the leaf (64: always)
#endif

namespace orr {

namespace {

// Orders the wave's LDS accesses around a hand-over between lanes (LDS
// requests of one wave are served in order; this keeps the compiler's order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Particles per row when k lanes open a leaf of cnt particles: the wave is
// split into g slots of 64/g lanes (g = 64 / k rounded down to a power of
// two), each slot one particle, each lane of a slot one opening lane; no
// wider than the leaf needs. g = 1: no packing.
__device__ __forceinline__ uint32_t pack_width(uint32_t k, uint32_t cnt) {
    if (k > ORR_PACK_KMAX) return 1u;
    uint32_t g = 64u >> (32u - __clz(k - 1u));  // 64 / (k rounded up to a power of two); k >= 1
    while (g > 1 && (g >> 1) >= cnt) g >>= 1;
    return g;
}

// A leaf opened by many lanes: its particles are staged in the wave's LDS
// (one coalesced load, one particle per lane) and every opening lane adds
// them in particle order, one broadcast LDS read per particle.
template <int kInv>
__device__ __forceinline__ void leaf_masked(const float4 *__restrict__ xs, uint32_t b, uint32_t cnt, bool opening,
                                            const float4 &xi, float eps2, float &ax, float &ay, float &az,
                                            float4 *src) {
    const uint32_t lane = __lane_id();
    for (uint32_t c0 = 0; c0 < cnt; c0 += 64) {
        const uint32_t cc = min(cnt - c0, 64u);
        if (lane < cc) src[lane] = xs[b + c0 + lane];
        wave_lds_sync();
        if (opening) {
            uint32_t j = 0;
            for (; j + 4u <= cc; j += 4u) {  // four reads in flight
                const float4 p0 = src[j], p1 = src[j + 1], p2 = src[j + 2], p3 = src[j + 3];
                add_term<kInv>(p0.w, p0.x - xi.x, p0.y - xi.y, p0.z - xi.z, eps2, ax, ay, az);
                add_term<kInv>(p1.w, p1.x - xi.x, p1.y - xi.y, p1.z - xi.z, eps2, ax, ay, az);
                add_term<kInv>(p2.w, p2.x - xi.x, p2.y - xi.y, p2.z - xi.z, eps2, ax, ay, az);
                add_term<kInv>(p3.w, p3.x - xi.x, p3.y - xi.y, p3.z - xi.z, eps2, ax, ay, az);
            }
            for (; j < cc; j++) {
                const float4 p = src[j];
                add_term<kInv>(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
            }
        }
        wave_lds_sync();
    }
}

// A leaf opened by the lanes of m_open, packed kG > 1 particles per row:
// lane (slot q, position r) computes the term product of the row's particle
// q for the r-th opening lane; each opening lane then adds its kG products of
// the row in particle order, so its sum is the one its own walk makes. Slots
// past the leaf's end hold +0 products, and adding +0 leaves every
// accumulator unchanged (an accumulator that starts at +0 never becomes -0
// under round-to-nearest), so the rows need no tail test. Per wave LDS:
// tgt = the opening lanes' positions, src = up to 64 of the leaf's particles,
// prod = one row of products.
template <int kInv, uint32_t kG>
__device__ __forceinline__ void leaf_packed(const float4 *__restrict__ xs, uint32_t b, uint32_t cnt, uint64_t m_open,
                                            bool opening, const float4 &xi, float eps2, float &ax, float &ay,
                                            float &az, float4 *tgt, float4 *src, float4 *prod) {
    constexpr uint32_t kSlot = 64u / kG;  // lanes per slot: opening lanes served per particle
    const uint32_t lane = __lane_id();
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m_open >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m_open, 0u));
    const uint32_t k = (uint32_t)__popcll(m_open);
    const uint32_t q = lane / kSlot, r = lane % kSlot;
    if (opening) tgt[rank] = xi;
    wave_lds_sync();
    const float4 t = r < k ? tgt[r] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (uint32_t c0 = 0; c0 < cnt; c0 += 64) {
        const uint32_t cc = min(cnt - c0, 64u);
        if (lane < cc) src[lane] = xs[b + c0 + lane];
        wave_lds_sync();
        for (uint32_t j0 = 0; j0 < cc; j0 += kG) {
            if (r < k) {
                float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (j0 + q < cc) {
                    const float4 p = src[j0 + q];
                    v = term_product<kInv>(p.w, p.x - t.x, p.y - t.y, p.z - t.z, eps2);
                }
                prod[lane] = v;
            }
            wave_lds_sync();
            if (opening) {
#pragma unroll
                for (uint32_t qq = 0; qq < kG; qq++) {
                    const float4 v = prod[qq * kSlot + rank];
                    ax += v.x;
                    ay += v.y;
                    az += v.z;
                }
            }
            wave_lds_sync();
        }
    }
}

// v + 1 on the lanes whose bit is set in mask, v elsewhere: one add with the
// mask as carry-in.
__device__ __forceinline__ uint32_t add_lane_bit(uint32_t v, uint64_t mask) {
    uint32_t r;
    uint64_t carry;
    __asm__("v_addc_co_u32_e64 %0, %1, 0, %2, %3" : "=v"(r), "=s"(carry) : "v"(v), "s"(mask));
    return r;
}

// A leaf opened by k <= 16 lanes, packed kG >= 4 particles per row as in
// leaf_packed, with the sums spread over lanes: the accumulator component c
// of opening lane r is carried by lane 16 c + r, which adds the row's kG
// products of that component in particle order (one add per product instead
// of three in the opening lane). The accumulators go to those lanes through
// LDS before the leaf and come back after it; every accumulator sees the same
// additions in the same order as its own lane would make.
template <int kInv, uint32_t kG>
__device__ __forceinline__ void leaf_chain(const float4 *__restrict__ xs, uint32_t b, uint32_t cnt, uint64_t m_open,
                                           bool opening, const float4 &xi, float eps2, float &ax, float &ay,
                                           float &az, float4 *tgt, float4 *src, float *prod, float4 *acc) {
    constexpr uint32_t kSlot = 64u / kG;  // >= 16 >= k
    const uint32_t lane = __lane_id();
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m_open >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m_open, 0u));
    const uint32_t k = (uint32_t)__popcll(m_open);
    const uint32_t q = lane / kSlot, r = lane % kSlot;
    const uint32_t cr = lane & 15u, cc = lane >> 4;  // chain lane: opening lane cr, component cc
    const bool chain = cr < k && cc < 3u;
    if (opening) {
        tgt[rank] = xi;
        acc[rank] = make_float4(ax, ay, az, 0.0f);
    }
    wave_lds_sync();
    float a = chain ? reinterpret_cast<const float *>(acc)[4u * cr + cc] : 0.0f;
    const float4 t = r < k ? tgt[r] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (uint32_t c0 = 0; c0 < cnt; c0 += 64) {
        const uint32_t n0 = min(cnt - c0, 64u);
        if (lane < n0) src[lane] = xs[b + c0 + lane];
        wave_lds_sync();
        for (uint32_t j0 = 0; j0 < n0; j0 += kG) {
            if (r < k) {
                float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (j0 + q < n0) {
                    const float4 p = src[j0 + q];
                    v = term_product<kInv>(p.w, p.x - t.x, p.y - t.y, p.z - t.z, eps2);
                }
                prod[r * kG + q] = v.x;
                prod[64u + r * kG + q] = v.y;
                prod[128u + r * kG + q] = v.z;
            }
            wave_lds_sync();
            if (chain) {
                const float *pc = prod + 64u * cc + cr * kG;
#pragma unroll
                for (uint32_t qq = 0; qq < kG; qq++) a += pc[qq];
            }
            wave_lds_sync();
        }
    }
    if (chain) reinterpret_cast<float *>(acc)[4u * cr + cc] = a;
    wave_lds_sync();
    if (opening) {
        const float4 v = acc[rank];
        ax = v.x;
        ay = v.y;
        az = v.z;
    }
    wave_lds_sync();
}

// Wave-private LDS of the packed leaf evaluation, for kWaves waves.
template <uint32_t kWaves>
struct WalkLdsT {
    float4 tgt[kWaves][64], src[kWaves][64], prod[kWaves][64], acc[kWaves][64];
};
using WalkLds = WalkLdsT<kWalkBlock / 64>;

// The terms of leaf [b, b + cnt) for the lanes of m_open (opening = this
// lane's bit of m_open), in particle order, with the path that suits the
// number of opening lanes: all lanes reading the staged particles when more
// than 32 open it, else rows packed across the wave (g particles per row).
template <int kInv, uint32_t kWaves>
__device__ __forceinline__ void leaf_terms(const float4 *__restrict__ xs, uint32_t b, uint32_t cnt, uint64_t m_open,
                                           bool opening, const float4 &xi, float eps2, float &ax, float &ay,
                                           float &az, WalkLdsT<kWaves> &lds, uint32_t wv) {
    const uint32_t g = pack_width((uint32_t)__popcll(m_open), cnt);
    if (g == 1) {
        leaf_masked<kInv>(xs, b, cnt, opening, xi, eps2, ax, ay, az, lds.src[wv]);
        return;
    }
#define ORR_LEAF_PACKED(G)                                                                                 \
    case G:                                                                                                \
        leaf_packed<kInv, G>(xs, b, cnt, m_open, opening, xi, eps2, ax, ay, az, lds.tgt[wv], lds.src[wv], \
                             lds.prod[wv]);                                                                \
        break;
#define ORR_LEAF_CHAIN(G)                                                                                 \
    case G:                                                                                               \
        leaf_chain<kInv, G>(xs, b, cnt, m_open, opening, xi, eps2, ax, ay, az, lds.tgt[wv], lds.src[wv], \
                            reinterpret_cast<float *>(lds.prod[wv]), lds.acc[wv]);                        \
        break;
    switch (g) {  // g >= 4: at most 16 opening lanes
        ORR_LEAF_PACKED(2)
        ORR_LEAF_CHAIN(4)
        ORR_LEAF_CHAIN(8)
        ORR_LEAF_CHAIN(16)
        ORR_LEAF_CHAIN(32)
        default:
            ORR_LEAF_CHAIN(64)
    }
#undef ORR_LEAF_PACKED
#undef ORR_LEAF_CHAIN
}

}  // namespace

}  // namespace orr
