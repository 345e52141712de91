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
#include <cstdlib>
#include <cstring>

#include "checked.h"
#include "orr_internal.h"
#include "term.h"
#include "schedule.h"
#include "walk_common.h"
#include "walk_leaf.h"

namespace orr {

namespace {

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

// kMin: the wave advances to the minimum of the lanes' `next` (every lane
// keeps its own next node, c + 1 after opening), found with a DPP
// reduction, instead of the select on the opening mask. Both rules give the
// same node sequence (the next node any lane wants is c + 1 if some lane
// opened c and escape[c] otherwise); kMin exists to measure the cost of the
// explicit reduction.
// kSplit (1, 2, 4, 8, 16): the target wave's 64 walks are shared by kSplit
// hardware waves. Each runs the whole traversal (node loads, opening tests of
// all 64 lanes, advance), so all of them step through the same nodes, and
// each adds the terms, accepted cells and opened leaves, of its own 64 /
// kSplit lanes only (lanes part * 64 / kSplit ..). A target's sum is made by
// one lane in its walk's order as before; the leaf and term work of a step is
// spread over kSplit SIMDs, for grids that leave most SIMDs idle.
// kPow2: theta^2 = 2^-e, and every node's s^2 times 2^e is a normal float
// (pow2_scale_ok): then s^2 < RN(theta^2 d^2) exactly when s^2 2^e < d^2, and
// s^2 2^e is the scalar integer sum s2_bits + s2_shift (s2_shift = e << 23),
// one scalar instruction in place of a vector multiply on every step. Proof:
// if 2^-e d^2 is a normal float (or 0), both sides compare the same real
// numbers scaled by 2^e; if it is not, it is below 2^-126 <= s^2, and both
// comparisons are false.
template <int kInv, bool kOff32, bool kMin, bool kPow2, uint32_t kSplit>
__device__ __forceinline__ void walk_coherent(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                              const uint32_t *__restrict__ perm, uint32_t i, uint32_t part,
                                              uint32_t n, uint32_t n_nodes, float eps2, float theta2,
                                              uint32_t s2_shift, const WalkOut &out, WalkLds &lds,
                                              const Check &ck) {
    static_assert(kSplit == 1 || kSplit == 2 || kSplit == 4 || kSplit == 8 || kSplit == 16, "split");
    constexpr uint32_t kOwn = 64u / kSplit;  // lanes whose terms this wave adds
    const uint64_t own_mask = kSplit == 1 ? ~0ull : ((1ull << kOwn) - 1ull) << (part * kOwn);
    const bool own = kSplit == 1 || __lane_id() / kOwn == part;
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
        const uint32_t esc = nd.t.x;  // > c: the build stores escape = max(escape, index + 1)
        const uint32_t c1 = c + 1;
        ORR_IF_CHECKED(if (!escape_ok(c, esc, n_nodes, ck.word)) break;)  // wave-uniform
        // A lane that did not accept at the wave's previous node wants exactly
        // the node the wave visits next (it opened that node, so it wants the
        // node after it, which is the smallest index any lane can want), so
        // `next` only changes when a lane accepts a cell: it then waits for
        // the escape. The lanes acting at c are those with next <= c.
        const bool active = next < c1;
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
        if (kSplit == 1) {
            if (active && far) {  // accept: monopole term, then wait for the escape
                add_term_r2<kInv>(mass_c, dx, dy, dz, d2 + eps2, ax, ay, az);
                pc += 1;
                next = esc;
            }
        } else {
            if (active && far && own) {  // accept, own lanes: the monopole term
                add_term_r2<kInv>(mass_c, dx, dy, dz, d2 + eps2, ax, ay, az);
                pc += 1;
            }
            next = active && far ? esc : next;  // every lane: wait for the escape
        }
        const bool opening = active && !far && own;  // own lanes opening c
        if (m_open) {
            nopen = add_lane_bit(nopen, m_open);
            const uint64_t m_mine = m_open & own_mask;  // the opening lanes whose terms this wave adds
            if (esc == c1 && m_mine && leaf_ok(nd.t.y, nd.t.z, ck)) {  // a leaf that some own lane opens
                const uint32_t b = nd.t.y, cnt = nd.t.z;
                leaf_terms<kInv>(xs, b, cnt, m_mine, opening, xi, eps2, ax, ay, az, lds, wv);
                if (opening) pp += cnt - ((i - b) < cnt ? 1u : 0u);
            }
        }
        if (kMin) {
            if (active && !far) next = c1;
            c = max(wave_min_u32(next), c1);  // the max only guards progress; the minimum exceeds c
        } else {
            // The smallest index any lane wants: c + 1 if some lane opened c
            // (a waiting lane wants the escape of a skipped ancestor of c, at
            // least escape[c]; for a leaf escape[c] = c + 1 anyway), else the
            // escape.
            c = m_open ? c1 : esc;
        }
    }
    if (valid && own) {
        const uint32_t dst = perm[i];
        if (checked_lt(dst, ck.n_particles, ck.word)) write_out(out, dst, ax, ay, az, pc + nopen, steps, pp, pc);
    }
}

// The walk schedule (which waves each XCD runs, longest first) is computed
// by the tree build (schedule.h).

// Eight waves per SIMD (at most 64 VGPRs): the occupancy the walk's issue
// rate needs; without the bound the unrolled leaf sums take more registers.
// The split variants run only on grids that fill at most half the wave
// slots, so they take the registers they need (at least 4 waves per SIMD)
// instead of spilling 30 of them to scratch.
template <bool kOff32, bool kMin, uint32_t kSplit>
__global__ __launch_bounds__(kWalkBlock) __attribute__((amdgpu_waves_per_eu(kSplit == 1 ? 8 : 4, 8))) void k_walk_coherent(const float4 *__restrict__ xs,
                                                              const NodeRec *__restrict__ nodes,
                                                              const DevParams *__restrict__ prm,
                                                              const uint32_t *__restrict__ perm, uint32_t n,
                                                              uint32_t max_nodes, float eps2, float theta2,
                                                              const uint32_t *__restrict__ order,
                                                              uint32_t n_waves, uint32_t wave0, uint32_t theta2_exp,
                                                              WalkOut out) {
    __shared__ WalkLds lds;
    uint32_t part;
    const uint32_t i = scheduled_target<kSplit>(order, n_waves, wave0, &part);  // walked if i < n
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const uint32_t sh = theta2_exp << 23;
    // the scaled comparison only in the production variant (uniform branches)
    constexpr bool kScaled = kOff32 && !kMin;
    const bool pow2 = kScaled && pow2_scale_ok(prm, theta2_exp);
    const Check ck = make_check(prm);
#define ORR_WALK(INV, POW2) \
    walk_coherent<INV, kOff32, kMin, POW2, kSplit>(xs, nodes, perm, i, part, n, n_nodes, eps2, theta2, sh, out, lds, ck)
    if (r2_cannot_overflow(prm, eps2)) {
        if (pow2)
            ORR_WALK(kInvFastNoClamp, kScaled);
        else
            ORR_WALK(kInvFastNoClamp, false);
    } else {
        if (pow2)
            ORR_WALK(kInvFast, kScaled);
        else
            ORR_WALK(kInvFast, false);
    }
#undef ORR_WALK
}

template <int kInv>
__device__ __forceinline__ void walk_independent(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                                 const uint32_t *__restrict__ perm, uint32_t i, uint32_t n_nodes,
                                                 float eps2, float theta2, const WalkOut &out, const Check &ck) {
    const float4 xi = xs[i];
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    uint32_t vown = 0, pp = 0, pc = 0;
    uint32_t c = 0;
    while (c < n_nodes) {
        const NodeRec nd = nodes[c];
        ORR_IF_CHECKED(if (!escape_ok(c, nd.t.x, n_nodes, ck.word)) break;)
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
            if (leaf_ok(b, cnt, ck)) {
                for (uint32_t j = b; j < b + cnt; j++) {
                    const float4 p = xs[j];
                    add_term<kInv>(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
                }
                pp += cnt - ((i - b) < cnt ? 1u : 0u);
            }
            c = esc;
        } else {
            c = c + 1;
        }
    }
    const uint32_t dst = perm[i];
    if (checked_lt(dst, ck.n_particles, ck.word)) write_out(out, dst, ax, ay, az, vown, vown, pp, pc);
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
    const Check ck = make_check(prm);
    if (r2_cannot_overflow(prm, eps2))
        walk_independent<kInvFastNoClamp>(xs, nodes, perm, i, n_nodes, eps2, theta2, out, ck);
    else
        walk_independent<kInvFast>(xs, nodes, perm, i, n_nodes, eps2, theta2, out, ck);
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

// Hardware waves per target wave of the coherent walk: grids of target waves
// that fill only part of the GPU's wave slots (256 CUs x 4 SIMDs x 8 waves)
// share each target wave's terms among 2 to 16 hardware waves (walk_coherent,
// kSplit), so that more SIMDs work on the same walks. Measured (walk medians,
// Plummer): 16 waves beat 8 up to 128 target waves (8,192 particles: 0.297
// against 0.324 ms) but not at 256 (16,384: 0.385 against 0.388, and uniform
// 16,384 0.216 against 0.196); 8 beat 4 up to 512 (16,384: 0.397 against
// 0.463, 32,768: 0.475 against 0.495).
#ifndef ORR_WALK_SPLIT_FORCE
#define ORR_WALK_SPLIT_FORCE 0
#endif
uint32_t walk_split(int64_t target_waves) {
    if (ORR_WALK_SPLIT_FORCE) return ORR_WALK_SPLIT_FORCE;
    constexpr int64_t kSlots = 256 * 4 * 8;
    if (16 * target_waves <= kSlots / 4) return 16;
    if (8 * target_waves <= kSlots / 2) return 8;
    if (4 * target_waves <= kSlots / 2) return 4;
    if (2 * target_waves <= kSlots / 2) return 2;
    return 1;
}

hipError_t launch_walk_t(const Workspace &ws, int mode, const WalkRange &rg, float eps2, float theta2,
                         const WalkOut &out, hipStream_t s) {
    const uint32_t nb = (uint32_t)ws.max_nodes;
    const uint32_t end = (uint32_t)(rg.first + rg.count);  // targets [first, end) are walked
    if (mode != kWalkIndependent) {
        const char *force = std::getenv("ORR_WALK_NODE_OFFSETS");  // "64": the large-tree path at any size
        const bool off32 = (uint64_t)ws.max_nodes * sizeof(NodeRec) <= 0xffffffffull &&
                           !(force && std::strcmp(force, "64") == 0);
        const int64_t nw = ceil_div(rg.count, (int64_t)64);
        // 8 XCD lists of up to L target waves each (scheduled_target)
        const int64_t L = (int64_t)(kScheduleRegions / 8) * ceil_div(nw, (int64_t)kScheduleRegions);
        const uint32_t split = mode == kWalkCoherentMin ? 1u : walk_split(nw);
        const unsigned cblocks = 8u * (unsigned)ceil_div(L * split, (int64_t)(kWalkBlock / 64));
        const uint32_t wave0 = (uint32_t)(rg.first / 64);
        const uint32_t e2 = theta2_pow2_exp(theta2);
#define ORR_COHERENT(OFF32, MIN, SPLIT)                                                                          \
    k_walk_coherent<OFF32, MIN, SPLIT><<<cblocks, kWalkBlock, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0], end, \
                                                                     nb, eps2, theta2, rg.order, (uint32_t)nw,  \
                                                                     wave0, e2, out)
        if (mode == kWalkCoherentMin) {
            if (off32)
                ORR_COHERENT(true, true, 1);
            else
                ORR_COHERENT(false, true, 1);
        } else if (!off32) {
            ORR_COHERENT(false, false, 1);
        } else if (split == 16) {
            ORR_COHERENT(true, false, 16);
        } else if (split == 8) {
            ORR_COHERENT(true, false, 8);
        } else if (split == 4) {
            ORR_COHERENT(true, false, 4);
        } else if (split == 2) {
            ORR_COHERENT(true, false, 2);
        } else {
            ORR_COHERENT(true, false, 1);
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
