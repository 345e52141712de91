// The two tree walks (enum TreeTraversal of the orrery solver page).
//
// Coherent walk (solver page, "The mitigation"; ADR-0029, Decision): one
// 64-lane wave walks one node index kept in a scalar register. The wave moves
// to the smallest node any lane's own walk wants: c + 1 if a lane opened c
// and escape[c] otherwise (a lane waiting at c skipped an ancestor of c, so
// it wants at least escape[c]). A lane that accepts c waits for escape[c]
// (`next`); every other lane wants exactly the wave's next node, so `next`
// changes only on acceptance and the lanes acting at c are those with
// next <= c. The advance is one scalar select on the mask of opening lanes.
// Node records are wave-uniform and come through scalar loads. An opened leaf
// is read once for all its opening lanes: its particles are staged in the
// wave's LDS with one coalesced load; when few lanes open it, their terms are
// also packed across the wave's lanes. Each XCD takes its target waves from
// its own list of the schedule (schedule.h), longest first; a range walk
// takes them from the schedule of its range.
//
// Independent walk (enum TreeTraversal, kIndependent): one lane per target,
// each following its own node index with per-lane vector loads; the measured
// baseline.
//
// Both add the same terms in the same order with the same float operations,
// so their accelerations are identical bit for bit and their visits_own,
// n_pp and n_pc equal the oracle's. Each lane handles one sorted target (a
// wave the 64 targets 64 w .. 64 w + 63); outputs go straight to the
// caller's order through perm (the scatter step of the performance page's
// "Where one evaluation goes" table).
#include "orr_internal.h"
#include "term.h"
#include "schedule.h"
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

// Smallest value over the wave's 64 lanes, wave-uniform: DPP minima within
// rows of 16 lanes (two quad permutations, two row rotations), two row
// broadcasts that carry the minimum to the last lane, then that lane's value.
// Each step is one v_min_u32 with a DPP source; rows outside row_mask keep
// their value. The s_nop before each step covers the wait a DPP read needs
// after a VALU write of the same register. Needs every lane active.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    __asm__ volatile(
        "s_nop 1\n\t"
        "v_min_u32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_min_u32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_min_u32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_min_u32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_min_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_min_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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

// Sorted targets of this lane's wave: block b runs on XCD b mod 8 and takes
// its waves from that XCD's list of the schedule, in block order (wave slot s
// of the XCD runs list entry s: targets 64 (wave0 + w) .. + 63 of the
// schedule's wave w, whose waves start at wave0). Slots past the list get the
// first target past the schedule's waves, which no lane walks.
__device__ __forceinline__ uint32_t scheduled_target(const uint32_t *__restrict__ order, uint32_t n_waves,
                                                     uint32_t wave0) {
    const uint32_t L = (kScheduleRegions / 8u) * ((n_waves + kScheduleRegions - 1u) / kScheduleRegions);
    const uint32_t x = blockIdx.x & 7u;
    const uint32_t s = (blockIdx.x >> 3) * (kWalkBlock / 64u) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t w = s < order[8u * L + x] ? min(order[x * L + s], n_waves) : n_waves;
    return (wave0 + w) * 64u + (threadIdx.x & 63u);
}

// Wave-private LDS of the packed leaf evaluation.
struct WalkLds {
    float4 tgt[kWalkBlock / 64][64], src[kWalkBlock / 64][64], prod[kWalkBlock / 64][64], acc[kWalkBlock / 64][64];
};

// kMin: the wave advances to the minimum of the lanes' `next` (every lane
// keeps its own next node, c + 1 after opening), found with a DPP
// reduction, instead of the select on the opening mask. Both rules give the
// same node sequence (the next node any lane wants is c + 1 if some lane
// opened c and escape[c] otherwise); kMin exists to measure the cost of the
// explicit reduction.
// kPow2: theta^2 = 2^-e, and every node's s^2 times 2^e is a normal float
// (pow2_scale_ok): then s^2 < RN(theta^2 d^2) exactly when s^2 2^e < d^2, and
// s^2 2^e is the scalar integer sum s2_bits + s2_shift (s2_shift = e << 23),
// one scalar instruction in place of a vector multiply on every step. Proof:
// if 2^-e d^2 is a normal float (or 0), both sides compare the same real
// numbers scaled by 2^e; if it is not, it is below 2^-126 <= s^2, and both
// comparisons are false.
template <int kInv, bool kOff32, bool kMin, bool kPow2>
__device__ __forceinline__ void walk_coherent(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                              const uint32_t *__restrict__ perm, uint32_t i, uint32_t n,
                                              uint32_t n_nodes, float eps2, float theta2, uint32_t s2_shift,
                                              const WalkOut &out, WalkLds &lds) {
    const bool valid = i < n;
    const float4 xi = valid ? xs[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    uint32_t next = valid ? 0u : n_nodes;  // lanes without a target never act
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    const uint32_t wv = threadIdx.x >> 6;
    uint32_t pp = 0, pc = 0, nopen = 0;  // visits_own = pc + nopen: every acting lane accepts or opens
    uint32_t steps = 0;  // wave-uniform: visits_stepped
    const char *node_bytes = reinterpret_cast<const char *>(nodes);
    uint32_t c = 0;
    while (c < n_nodes) {
        c = __builtin_amdgcn_readfirstlane(c);
        steps += 1;
        // One scalar load of 32 bytes; kOff32: at a 32-bit byte offset from
        // the array (the launch checks that 32 n_nodes fits), which saves the
        // 64-bit address arithmetic of every step.
        const NodeRec nd = kOff32 ? *reinterpret_cast<const NodeRec *>(node_bytes + (c << 5)) : nodes[c];
        const uint32_t esc = max(nd.t.x, c + 1);  // a well-formed tree has escape > c; never step back
        // A lane that did not accept at the wave's previous node wants exactly
        // the node the wave visits next (it opened that node, so it wants the
        // node after it, which is the smallest index any lane can want), so
        // `next` only changes when a lane accepts a cell: it then waits for
        // the escape. The lanes acting at c are those with next <= c.
        const bool active = next <= c;
        const float dx = nd.g.x - xi.x, dy = nd.g.y - xi.y, dz = nd.g.z - xi.z;
        const float d2 = (dx * dx + dy * dy) + dz * dz;
        // s/d < theta: s^2 < theta^2 d^2, or s^2 2^e < d^2 (kPow2)
        const float lhs = kPow2 ? __uint_as_float(nd.t.w + s2_shift) : __uint_as_float(nd.t.w);
        const float rhs = kPow2 ? d2 : theta2 * d2;
        const bool far = lhs < rhs;
        // Lanes opening c, from the two comparison masks.
        const uint64_t m_open =
            __builtin_amdgcn_ballot_w64(active) & ~__builtin_amdgcn_fcmpf(lhs, rhs, 4 /* ordered < */);
        // Divergent branches below are skipped when no lane takes them.
        float mass_c = nd.g.w;
        __asm__ volatile("" : "+s"(mass_c));  // keeps the node mass in its register rather than loading it again
        if (active && far) {  // accept: monopole term, then wait for the escape
            add_term_r2<kInv>(mass_c, dx, dy, dz, d2 + eps2, ax, ay, az);
            pc += 1;
            next = esc;
        }
        const bool opening = active && !far;
        if (m_open) {
            nopen = add_lane_bit(nopen, m_open);
            if (esc == c + 1) {  // a leaf that some lane opens
                const uint32_t b = nd.t.y, cnt = nd.t.z;
                const uint32_t g = pack_width((uint32_t)__popcll(m_open), cnt);
                if (g == 1) {
                    leaf_masked<kInv>(xs, b, cnt, opening, xi, eps2, ax, ay, az, lds.src[wv]);
                } else {
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
                if (opening) pp += cnt - ((i - b) < cnt ? 1u : 0u);
            }
        }
        if (kMin) {
            if (opening) next = c + 1;
            c = max(wave_min_u32(next), c + 1);  // the max only guards progress; the minimum exceeds c
        } else {
            // The smallest index any lane wants: c + 1 if some lane opened c
            // (a waiting lane wants the escape of a skipped ancestor of c, at
            // least escape[c]; for a leaf escape[c] = c + 1 anyway), else the
            // escape.
            c = m_open ? c + 1 : esc;
        }
    }
    if (valid) write_out(out, perm[i], ax, ay, az, pc + nopen, steps, pp, pc);
}

// The walk schedule (which waves each XCD runs, longest first) is computed
// by the tree build (schedule.h).

// Eight waves per SIMD (at most 64 VGPRs): the occupancy the walk's issue
// rate needs; without the bound the unrolled leaf sums take more registers.
template <bool kOff32, bool kMin>
__global__ __launch_bounds__(kWalkBlock) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_walk_coherent(const float4 *__restrict__ xs,
                                                              const NodeRec *__restrict__ nodes,
                                                              const DevParams *__restrict__ prm,
                                                              const uint32_t *__restrict__ perm, uint32_t n,
                                                              uint32_t max_nodes, float eps2, float theta2,
                                                              const uint32_t *__restrict__ order,
                                                              uint32_t n_waves, uint32_t wave0, uint32_t theta2_exp,
                                                              WalkOut out) {
    __shared__ WalkLds lds;
    const uint32_t i = scheduled_target(order, n_waves, wave0);  // walked if i < n
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const uint32_t sh = theta2_exp << 23;
    // the scaled comparison only in the production variant (uniform branches)
    constexpr bool kScaled = kOff32 && !kMin;
    const bool pow2 = kScaled && pow2_scale_ok(prm, theta2_exp);
    if (r2_cannot_overflow(prm, eps2)) {
        if (pow2)
            walk_coherent<kInvFastNoClamp, kOff32, kMin, kScaled>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh,
                                                                  out, lds);
        else
            walk_coherent<kInvFastNoClamp, kOff32, kMin, false>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh,
                                                                out, lds);
    } else {
        if (pow2)
            walk_coherent<kInvFast, kOff32, kMin, kScaled>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out,
                                                           lds);
        else
            walk_coherent<kInvFast, kOff32, kMin, false>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out,
                                                         lds);
    }
}

template <int kInv>
__device__ __forceinline__ void walk_independent(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                                 const uint32_t *__restrict__ perm, uint32_t i, uint32_t n_nodes,
                                                 float eps2, float theta2, const WalkOut &out) {
    const float4 xi = xs[i];
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    uint32_t vown = 0, pp = 0, pc = 0;
    uint32_t c = 0;
    while (c < n_nodes) {
        const NodeRec nd = nodes[c];
        const uint32_t esc = max(nd.t.x, c + 1);  // a well-formed tree has escape > c; never step back
        const float dx = nd.g.x - xi.x, dy = nd.g.y - xi.y, dz = nd.g.z - xi.z;
        const float d2 = (dx * dx + dy * dy) + dz * dz;
        vown += 1;
        if (__uint_as_float(nd.t.w) < theta2 * d2) {
            add_term_r2<kInv>(nd.g.w, dx, dy, dz, d2 + eps2, ax, ay, az);
            pc += 1;
            c = esc;
        } else if (esc == c + 1) {
            const uint32_t b = nd.t.y, cnt = nd.t.z;
            for (uint32_t j = b; j < b + cnt; j++) {
                const float4 p = xs[j];
                add_term<kInv>(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
            }
            pp += cnt - ((i - b) < cnt ? 1u : 0u);
            c = esc;
        } else {
            c = c + 1;
        }
    }
    write_out(out, perm[i], ax, ay, az, vown, vown, pp, pc);
}

__global__ __launch_bounds__(kWalkBlock) void k_walk_independent(const float4 *__restrict__ xs,
                                                                 const NodeRec *__restrict__ nodes,
                                                                 const DevParams *__restrict__ prm,
                                                                 const uint32_t *__restrict__ perm, uint32_t first,
                                                                 uint32_t n, uint32_t max_nodes, float eps2,
                                                                 float theta2, WalkOut out) {
    const uint32_t i = first + xcd_block(blockIdx.x, gridDim.x) * kWalkBlock + threadIdx.x;
    if (i >= n) return;
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    if (r2_cannot_overflow(prm, eps2))
        walk_independent<kInvFastNoClamp>(xs, nodes, perm, i, n_nodes, eps2, theta2, out);
    else
        walk_independent<kInvFast>(xs, nodes, perm, i, n_nodes, eps2, theta2, out);
}

// Self-check over the float bit patterns [first, first + count): the cube of
// inv_sqrt_rn (all the term uses) against the cube of the IEEE operations.
__global__ __launch_bounds__(256) void k_selftest_inv_sqrt(uint32_t first, uint64_t count,
                                                           unsigned long long *mismatches, uint32_t *examples) {
    const uint64_t stride = (uint64_t)gridDim.x * 256u;
    for (uint64_t k = (uint64_t)blockIdx.x * 256u + threadIdx.x; k < count; k += stride) {
        const uint32_t bits = first + (uint32_t)k;
        const float x = __uint_as_float(bits);
        const float r = 1.0f / sqrtf(x), y = inv_sqrt_rn(x);
        const float ref = (r * r) * r, got = (y * y) * y;
        if (__float_as_uint(got) != __float_as_uint(ref)) {
            const unsigned long long old = atomicAdd(mismatches, 1ull);
            if (old < 8) examples[old] = bits;
        }
    }
}

__global__ void k_zero_u64(unsigned long long *p) { *p = 0ull; }

// e with theta2 = 2^-e exactly, 0 <= e <= 126; kNotPow2 otherwise.
constexpr uint32_t kNotPow2 = 0xffffffffu;
uint32_t theta2_pow2_exp(float theta2) {
    if (!(theta2 > 0.0f && theta2 <= 1.0f)) return kNotPow2;
    int ex = 0;
    const float m = std::frexp(theta2, &ex);  // theta2 = m 2^ex, m in [0.5, 1)
    if (m != 0.5f || 1 - ex > 126) return kNotPow2;
    return (uint32_t)(1 - ex);
}

hipError_t launch_walk_t(const Workspace &ws, int mode, const WalkRange &rg, float eps2, float theta2,
                         const WalkOut &out, hipStream_t s) {
    const uint32_t nb = (uint32_t)ws.max_nodes;
    const uint32_t end = (uint32_t)(rg.first + rg.count);  // targets [first, end) are walked
    if (mode != kWalkIndependent) {
        const bool off32 = (uint64_t)ws.max_nodes * sizeof(NodeRec) <= 0xffffffffull;
        const int64_t nw = ceil_div(rg.count, (int64_t)64);
        // 8 XCD lists of up to L waves each (scheduled_target)
        const int64_t L = (int64_t)(kScheduleRegions / 8) * ceil_div(nw, (int64_t)kScheduleRegions);
        const unsigned cblocks = 8u * (unsigned)ceil_div(L, (int64_t)(kWalkBlock / 64));
        const uint32_t wave0 = (uint32_t)(rg.first / 64);
        const uint32_t e2 = theta2_pow2_exp(theta2);
#define ORR_COHERENT(OFF32, MIN)                                                                                  \
    k_walk_coherent<OFF32, MIN><<<cblocks, kWalkBlock, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0], end, nb, \
                                                                     eps2, theta2, rg.order, (uint32_t)nw, wave0,  \
                                                                     e2, out)
        if (mode == kWalkCoherentMin) {
            if (off32)
                ORR_COHERENT(true, true);
            else
                ORR_COHERENT(false, true);
        } else if (off32) {
            ORR_COHERENT(true, false);
        } else {
            ORR_COHERENT(false, false);
        }
#undef ORR_COHERENT
    } else {
        const unsigned blocks = (unsigned)ceil_div(rg.count, (int64_t)kWalkBlock);
        k_walk_independent<<<blocks, kWalkBlock, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0],
                                                                (uint32_t)rg.first, end, nb, eps2, theta2, out);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_walk(const Workspace &ws, int mode, float eps2, float theta2, float *acc,
                       uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                       hipStream_t s) {
    return launch_walk_range(ws, mode, WalkRange{0, ws.n, ws.wave_order}, eps2, theta2, acc, visits_own,
                             visits_stepped, n_pp, n_pc, s);
}

hipError_t launch_walk_range(const Workspace &ws, int mode, const WalkRange &rg, float eps2, float theta2,
                             float *acc, uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                             uint32_t *n_pc, hipStream_t s) {
    const WalkOut out{acc, visits_own, visits_stepped, n_pp, n_pc};
    return launch_walk_t(ws, mode, rg, eps2, theta2, out, s);
}

hipError_t launch_selftest_inv_sqrt(uint32_t first, uint64_t count, unsigned long long *mismatches,
                                    uint32_t *examples, hipStream_t s) {
    k_zero_u64<<<1, 1, 0, s>>>(mismatches);
    const uint64_t blocks = std::min<uint64_t>(std::max<uint64_t>(1, ceil_div((int64_t)count, 256)), 8192);
    k_selftest_inv_sqrt<<<(unsigned)blocks, 256, 0, s>>>(first, count, mismatches, examples);
    return hipGetLastError();
}

}  // namespace orr
