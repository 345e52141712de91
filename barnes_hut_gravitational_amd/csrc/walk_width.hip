// The coherent walk at other coherence widths, with the production walk's
// machinery (node records through scalar loads, opened leaves staged in LDS
// and packed across the wave), for the sub-group width question of the
// orrery pages (performance page, "The sub-group width": 16 against 32
// lanes, and whether a width of 64 would pay; ADR-0029, "Alternatives
// considered": coherence across a whole work-group).
//
// Width 32, k_walk_halves: a wave holds two groups of 32 consecutive sorted
// targets (lanes 0-31 and 32-63), each with its own node index in a scalar
// register. Every iteration steps both groups at once: two scalar record
// loads, per-lane selects of the half's record, one opening test over the
// wave, one advance per half, the opened leaves of each half in turn (the
// whole wave helps with either). A group steps through the union of its 32
// members' walks.
//
// Widths 128 and 256, k_walk_team: 2 or 4 waves of one work-group walk one
// node index. Each wave tests its own 64 lanes; whether any lane of the
// work-group opens the node is agreed through LDS at one barrier per step,
// and every wave then moves to c + 1 or the escape. A work-group steps
// through the union of its 128 or 256 members' walks.
//
// In both, each target sums exactly the nodes its own walk visits in walk
// order with the operations of term.h, so acc, visits_own, n_pp and n_pc are
// those of the 64-lane walk bit for bit; visits_stepped is the size of the
// union over the target's group of the given width.
#include "checked.h"
#include "orr_internal.h"
#include "term.h"
#include "schedule.h"
#include "walk_common.h"
#include "walk_leaf.h"

namespace orr {

namespace {

__device__ __forceinline__ NodeRec node_at(const NodeRec *__restrict__ nodes, uint32_t c) {
    return *reinterpret_cast<const NodeRec *>(reinterpret_cast<const char *>(nodes) + ((uint64_t)c << 5));
}

// s^2 < theta^2 d^2, or s^2 2^e < d^2 when kPow2 (see the production walk)
template <bool kPow2>
__device__ __forceinline__ bool opening_far(uint32_t s2_bits, uint32_t s2_shift, float theta2, float d2) {
    return kPow2 ? __uint_as_float(s2_bits + s2_shift) < d2 : __uint_as_float(s2_bits) < theta2 * d2;
}

// Two 32-target groups per wave (lanes 0-31 and 32-63), each with its own
// node index: the half-wave coherence of the pages' sub-groups at width 32.
// A lane's `next` is its own walk's next node within its half (the rules of
// the production walk, per half). A finished half loads record 0 and acts
// nowhere.
template <int kInv, bool kPow2>
__device__ __forceinline__ void walk_halves(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                            const uint32_t *__restrict__ perm, uint32_t i, uint32_t n,
                                            uint32_t n_nodes, float eps2, float theta2, uint32_t s2_shift,
                                            const WalkOut &out, WalkLds &lds, const Check &ck) {
    constexpr uint64_t kLo = 0x00000000ffffffffull, kHi = ~kLo;
    const bool valid = i < n;
    const bool hi = __lane_id() >= 32u;
    const float4 xi = valid ? xs[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    uint32_t next = valid ? 0u : n_nodes;  // lanes without a target never act
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    const uint32_t wv = threadIdx.x >> 6;
    uint32_t pp = 0, pc = 0, nopen = 0;
    uint32_t steps_lo = 0, steps_hi = 0;  // wave-uniform: each half's visits_stepped
    uint32_t c_lo = 0, c_hi = 0;
    while (c_lo < n_nodes || c_hi < n_nodes) {
        c_lo = __builtin_amdgcn_readfirstlane(c_lo);
        c_hi = __builtin_amdgcn_readfirstlane(c_hi);
        const bool run_lo = c_lo < n_nodes, run_hi = c_hi < n_nodes;
        steps_lo += run_lo ? 1u : 0u;
        steps_hi += run_hi ? 1u : 0u;
        const NodeRec a = node_at(nodes, run_lo ? c_lo : 0u);
        const NodeRec b = node_at(nodes, run_hi ? c_hi : 0u);
        // this lane's half: its node and its record, selected per lane
        const uint32_t c_me = hi ? c_hi : c_lo;
        const bool active = (hi ? run_hi : run_lo) && next <= c_me;
        const float gx = hi ? b.g.x : a.g.x, gy = hi ? b.g.y : a.g.y, gz = hi ? b.g.z : a.g.z;
        const float gm = hi ? b.g.w : a.g.w;
        const uint32_t s2b = hi ? b.t.w : a.t.w, esc_me = hi ? b.t.x : a.t.x;
        const float dx = gx - xi.x, dy = gy - xi.y, dz = gz - xi.z;
        const float d2 = (dx * dx + dy * dy) + dz * dz;
        const bool far = opening_far<kPow2>(s2b, s2_shift, theta2, d2);
        const uint64_t m_open = __builtin_amdgcn_ballot_w64(active && !far);
        if (active && far) {  // accept: monopole term, then wait for the escape
            add_term_r2<kInv>(gm, dx, dy, dz, d2 + eps2, ax, ay, az);
            pc += 1;
            next = esc_me;
        }
        const bool opening = active && !far;
        if (m_open) {
            nopen = add_lane_bit(nopen, m_open);
            // a leaf opened by lanes of the low half, then one of the high half
            // (one copy of the leaf code, run for each half in turn)
#pragma unroll 1
            for (uint32_t h = 0; h < 2u; h++) {
                const uint64_t m_h = m_open & (h ? kHi : kLo);
                const uint32_t esc_h = h ? b.t.x : a.t.x, c_h = h ? c_hi : c_lo;
                if (m_h && esc_h == c_h + 1u && leaf_ok(h ? b.t.y : a.t.y, h ? b.t.z : a.t.z, ck)) {
                    const uint32_t lb = h ? b.t.y : a.t.y, lc = h ? b.t.z : a.t.z;
                    const bool mine = opening && (hi == (h == 1u));
                    leaf_terms<kInv>(xs, lb, lc, m_h, mine, xi, eps2, ax, ay, az, lds, wv);
                    if (mine) pp += lc - ((i - lb) < lc ? 1u : 0u);
                }
            }
        }
        // per half: c + 1 if a lane of the half opened c, else the escape (a
        // half ends at a bad escape in the checked build)
        ORR_IF_CHECKED(const bool bad_lo = run_lo && !escape_ok(c_lo, a.t.x, n_nodes, ck.word);
                       const bool bad_hi = run_hi && !escape_ok(c_hi, b.t.x, n_nodes, ck.word);)
        if (run_lo) c_lo = (m_open & kLo) ? c_lo + 1u : a.t.x;
        if (run_hi) c_hi = (m_open & kHi) ? c_hi + 1u : b.t.x;
        ORR_IF_CHECKED(if (bad_lo) c_lo = n_nodes; if (bad_hi) c_hi = n_nodes;)
    }
    if (valid) {
        const uint32_t dst = perm[i];
        if (checked_lt(dst, ck.n_particles, ck.word))
            write_out(out, dst, ax, ay, az, pc + nopen, hi ? steps_hi : steps_lo, pp, pc);
    }
}

// Waves in the production walk's schedule (each wave 64 consecutive sorted
// targets, taken from its XCD's list, longest first), so that width 32 and
// width 64 differ in the coherence width and what it costs: the per-lane
// record selects and the second node index need 80 registers, so 6 waves
// per SIMD run instead of the production walk's 8 (at 8 the registers would
// spill).
__global__ __launch_bounds__(kWalkBlock) __attribute__((amdgpu_waves_per_eu(6, 6))) void k_walk_halves(const float4 *__restrict__ xs,
                                                            const NodeRec *__restrict__ nodes,
                                                            const DevParams *__restrict__ prm,
                                                            const uint32_t *__restrict__ perm, uint32_t n,
                                                            uint32_t max_nodes, float eps2, float theta2,
                                                            const uint32_t *__restrict__ order, uint32_t n_waves,
                                                            uint32_t theta2_exp, WalkOut out) {
    __shared__ WalkLds lds;
    uint32_t part;
    const uint32_t i = scheduled_target<1>(order, n_waves, 0u, &part);
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const uint32_t sh = theta2_exp << 23;
    const bool pow2 = pow2_scale_ok(prm, theta2_exp);
    const Check ck = make_check(prm);
    if (r2_cannot_overflow(prm, eps2)) {
        if (pow2)
            walk_halves<kInvFastNoClamp, true>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out, lds, ck);
        else
            walk_halves<kInvFastNoClamp, false>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out, lds, ck);
    } else {
        walk_halves<kInvFast, false>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out, lds, ck);
    }
}

// kTeam waves (one work-group) walk one node index. flags: three LDS words,
// used round-robin, one per step: a wave with an opening lane writes 1 into
// the step's word; after the barrier every wave reads it. The word of step
// t + 1 is cleared during step t: its last readers read it during step t - 2,
// before the barrier of step t - 1, which every wave has passed by then, and
// its next writers write it after the barrier of step t.
template <int kInv, bool kPow2, uint32_t kTeam>
__device__ __forceinline__ void walk_team(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                          const uint32_t *__restrict__ perm, uint32_t i, uint32_t n,
                                          uint32_t n_nodes, float eps2, float theta2, uint32_t s2_shift,
                                          const WalkOut &out, WalkLdsT<kTeam> &lds, volatile uint32_t *flags,
                                          const Check &ck) {
    const bool valid = i < n;
    const float4 xi = valid ? xs[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    uint32_t next = valid ? 0u : n_nodes;
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    const uint32_t wv = threadIdx.x >> 6;
    uint32_t pp = 0, pc = 0, nopen = 0;
    uint32_t steps = 0, slot = 0;  // block-uniform: visits_stepped; slot = steps mod 3
    uint32_t c = 0;
    while (c < n_nodes) {  // c is the same in every wave of the work-group
        c = __builtin_amdgcn_readfirstlane(c);
        steps += 1;
        const NodeRec nd = node_at(nodes, c);
        const uint32_t esc = nd.t.x, c1 = c + 1u;
        const bool active = next < c1;
        const float dx = nd.g.x - xi.x, dy = nd.g.y - xi.y, dz = nd.g.z - xi.z;
        const float d2 = (dx * dx + dy * dy) + dz * dz;
        const bool far = opening_far<kPow2>(nd.t.w, s2_shift, theta2, d2);
        const uint64_t m_open = __builtin_amdgcn_ballot_w64(active && !far);
        float mass_c = nd.g.w;
        __asm__ volatile("" : "+s"(mass_c));
        if (active && far) {
            add_term_r2<kInv>(mass_c, dx, dy, dz, d2 + eps2, ax, ay, az);
            pc += 1;
            next = esc;
        }
        const bool opening = active && !far;
        if (m_open) {
            nopen = add_lane_bit(nopen, m_open);
            if (esc == c1 && leaf_ok(nd.t.y, nd.t.z, ck)) {
                leaf_terms<kInv>(xs, nd.t.y, nd.t.z, m_open, opening, xi, eps2, ax, ay, az, lds, wv);
                if (opening) pp += nd.t.z - ((i - nd.t.y) < nd.t.z ? 1u : 0u);
            }
        }
        const uint32_t slot1 = slot == 2u ? 0u : slot + 1u;
        if (__lane_id() == 0u) {
            if (m_open) flags[slot] = 1u;
            if (wv == 0u) flags[slot1] = 0u;
        }
        __syncthreads();
        // the same word for every lane: readfirstlane makes the loop's exit
        // uniform for the compiler too, so its barrier stays in uniform
        // control flow
        const uint32_t any = __builtin_amdgcn_readfirstlane(flags[slot]);
        // every wave reads the same record, so all end together at a bad
        // escape (checked build)
        c = !escape_ok(c, esc, n_nodes, ck.word) ? n_nodes : any ? c1 : esc;
        slot = slot1;
    }
    if (valid) {
        const uint32_t dst = perm[i];
        if (checked_lt(dst, ck.n_particles, ck.word)) write_out(out, dst, ax, ay, az, pc + nopen, steps, pp, pc);
    }
}

template <uint32_t kTeam>
__global__ __launch_bounds__(64 * kTeam) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_walk_team(const float4 *__restrict__ xs,
                                                          const NodeRec *__restrict__ nodes,
                                                          const DevParams *__restrict__ prm,
                                                          const uint32_t *__restrict__ perm, uint32_t n,
                                                          uint32_t max_nodes, float eps2, float theta2,
                                                          uint32_t theta2_exp, WalkOut out) {
    __shared__ WalkLdsT<kTeam> lds;
    __shared__ uint32_t flags[3];
    const uint32_t i = xcd_block(blockIdx.x, gridDim.x) * (64u * kTeam) + threadIdx.x;
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const uint32_t sh = theta2_exp << 23;
    const bool pow2 = pow2_scale_ok(prm, theta2_exp);
    const Check ck = make_check(prm);
    if (threadIdx.x < 3u) flags[threadIdx.x] = 0u;
    __syncthreads();
    if (r2_cannot_overflow(prm, eps2)) {
        if (pow2)
            walk_team<kInvFastNoClamp, true, kTeam>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out, lds,
                                                   flags, ck);
        else
            walk_team<kInvFastNoClamp, false, kTeam>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out, lds,
                                                    flags, ck);
    } else {
        walk_team<kInvFast, false, kTeam>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, sh, out, lds, flags, ck);
    }
}

}  // namespace

hipError_t launch_walk_width(const Workspace &ws, int width, float eps2, float theta2, float *acc,
                             uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                             hipStream_t s) {
    const WalkOut out{acc, visits_own, visits_stepped, n_pp, n_pc};
    const uint32_t n = (uint32_t)ws.n, nb = (uint32_t)ws.max_nodes;
    const uint32_t e2 = theta2_pow2_exp(theta2);
    // node records are read at 32-bit byte offsets
    if ((uint64_t)ws.max_nodes * sizeof(NodeRec) > 0xffffffffull) return hipErrorInvalidValue;
    switch (width) {
        case 32: {
            // 8 XCD lists of up to L target waves each (scheduled_target)
            const int64_t L = (int64_t)(kScheduleRegions / 8) * ceil_div(ws.n_waves, (int64_t)kScheduleRegions);
            const unsigned blocks = 8u * (unsigned)ceil_div(L, (int64_t)(kWalkBlock / 64));
            k_walk_halves<<<blocks, kWalkBlock, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0], n, nb, eps2, theta2,
                                                        ws.wave_order, (uint32_t)ws.n_waves, e2, out);
            break;
        }
        case 64:
            return launch_walk(ws, kWalkCoherent, eps2, theta2, acc, visits_own, visits_stepped, n_pp, n_pc, s);
        case 128:
            k_walk_team<2><<<(unsigned)ceil_div(ws.n, 128), 128, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0],
                                                                              n, nb, eps2, theta2, e2, out);
            break;
        case 256:
            k_walk_team<4><<<(unsigned)ceil_div(ws.n, 256), 256, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0],
                                                                              n, nb, eps2, theta2, e2, out);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace orr
