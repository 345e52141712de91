// Walks for the coherence-width questions of the orrery pages: the masked
// walk with groups of 1, 2, ..., 64 targets sharing one node index ("The
// sub-group width" of the performance page), and the descend-together walk
// that ADR-0029 rejects ("Alternatives considered"). Both use per-lane vector
// loads; the production walks are in walk.hip.
#include "checked.h"
#include "orr_internal.h"
#include "term.h"
#include "walk_common.h"

namespace orr {

namespace {

// Walk of one target whose group of kW consecutive lanes (kW = 1..64, a
// power of two) shares one node index: the sub-group of the solver page at
// any width ("The sub-group width" of the performance page measures 16 and
// 32 lanes). The group steps through the union of its members' walks with
// the advance rule of the coherent walk applied to the group's lanes only.
// The node index is a vector register, equal across the group; node records
// and leaf particles come through per-lane vector loads (the lanes of a group
// read the same addresses). kW = 1 is the independent walk; kW = 64 is the
// coherent walk with vector instead of scalar loads. The sums and all counts
// except visits_stepped are the same for every width.
// kDescend: the alternative ADR-0029 rejects ("Alternatives considered"),
// the published warp-coherent traversal: the group opens a node when any
// member would and every member descends with it, so a target's sum depends
// on its group; every member acts at every node the group visits.
template <uint32_t kW, bool kDescend, int kInv>
__device__ __forceinline__ void walk_grouped(const float4 *__restrict__ xs, const NodeRec *__restrict__ nodes,
                                             const uint32_t *__restrict__ perm, uint32_t i, uint32_t n,
                                             uint32_t n_nodes, float eps2, float theta2, const WalkOut &out,
                                             const Check &ck) {
    static_assert(kW >= 1 && kW <= 64 && (kW & (kW - 1)) == 0, "group width");
    const bool valid = i < n;
    const float4 xi = valid ? xs[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    uint32_t next = valid ? 0u : n_nodes;  // lanes without a target never act
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    uint32_t pp = 0, pc = 0, nopen = 0, steps = 0;
    const uint32_t first = __lane_id() & ~(kW - 1);  // first lane of this lane's group
    const uint64_t gmask = kW == 64 ? ~0ull : ((1ull << kW) - 1ull);
    uint32_t c = 0;  // the group's node
    while (__builtin_amdgcn_ballot_w64(c < n_nodes)) {
        if (c < n_nodes) {
            steps += 1;
            const NodeRec nd = nodes[c];
            ORR_IF_CHECKED(if (!escape_ok(c, nd.t.x, n_nodes, ck.word)) {  // the same in the whole group
                c = n_nodes;
                continue;
            })
            const uint32_t esc = max(nd.t.x, c + 1);  // a well-formed tree has escape > c; never step back
            const float dx = nd.g.x - xi.x, dy = nd.g.y - xi.y, dz = nd.g.z - xi.z;
            const float d2 = (dx * dx + dy * dy) + dz * dz;
            const bool far = __uint_as_float(nd.t.w) < theta2 * d2;  // s/d < theta
            if (kDescend) {
                // The group opens c if any member with a target would; then
                // every member descends (at a leaf, sums its particles),
                // else every member adds c's term and the group skips c.
                const uint64_t opening = __builtin_amdgcn_ballot_w64(valid && !far);
                if ((opening >> first) & gmask) {
                    if (valid) {
                        nopen += 1;
                        if (esc == c + 1 && leaf_ok(nd.t.y, nd.t.z, ck)) {
                            const uint32_t b = nd.t.y, cnt = nd.t.z;
                            for (uint32_t j = b; j < b + cnt; j++) {
                                const float4 p = xs[j];
                                add_term<kInv>(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
                            }
                            pp += cnt - ((i - b) < cnt ? 1u : 0u);
                        }
                    }
                    c = c + 1;
                } else {
                    if (valid) {
                        add_term_r2<kInv>(nd.g.w, dx, dy, dz, d2 + eps2, ax, ay, az);
                        pc += 1;
                    }
                    c = esc;
                }
                continue;
            }
            const bool active = next == c;
            if (active && far) {  // accept: monopole term, then wait for the escape
                add_term_r2<kInv>(nd.g.w, dx, dy, dz, d2 + eps2, ax, ay, az);
                pc += 1;
                next = esc;
            }
            if (active && !far) {
                nopen += 1;
                if (esc == c + 1) {  // an opened leaf: its particles in sorted order
                    const uint32_t b = nd.t.y, cnt = nd.t.z;
                    if (leaf_ok(b, cnt, ck)) {
                        for (uint32_t j = b; j < b + cnt; j++) {
                            const float4 p = xs[j];
                            add_term<kInv>(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
                        }
                        pp += cnt - ((i - b) < cnt ? 1u : 0u);
                    }
                    next = esc;
                } else {
                    next = c + 1;
                }
            }
            // The smallest index a lane of the group wants: c + 1 if one of
            // them opened an internal c (waiting lanes want at least the
            // escape), else the escape, which is c + 1 for a leaf.
            const uint64_t down = __builtin_amdgcn_ballot_w64(next == c + 1);
            c = ((down >> first) & gmask) ? c + 1 : esc;
        }
    }
    if (valid) {
        const uint32_t dst = perm[i];
        if (checked_lt(dst, ck.n_particles, ck.word)) write_out(out, dst, ax, ay, az, pc + nopen, steps, pp, pc);
    }
}

template <uint32_t kW, bool kDescend>
__global__ __launch_bounds__(kWalkBlock) void k_walk_grouped(const float4 *__restrict__ xs,
                                                             const NodeRec *__restrict__ nodes,
                                                             const DevParams *__restrict__ prm,
                                                             const uint32_t *__restrict__ perm, uint32_t n,
                                                             uint32_t max_nodes, float eps2, float theta2,
                                                             WalkOut out) {
    const uint32_t i = xcd_block(blockIdx.x, gridDim.x) * kWalkBlock + threadIdx.x;
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const Check ck = make_check(prm);
    if (r2_cannot_overflow(prm, eps2))
        walk_grouped<kW, kDescend, kInvFastNoClamp>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, out, ck);
    else
        walk_grouped<kW, kDescend, kInvFast>(xs, nodes, perm, i, n, n_nodes, eps2, theta2, out, ck);
}

}  // namespace

template <bool kDescend>
hipError_t launch_walk_grouped_t(const Workspace &ws, int width, float eps2, float theta2, const WalkOut &out,
                                 hipStream_t s) {
    const uint32_t n = (uint32_t)ws.n;
    const uint32_t nb = (uint32_t)ws.max_nodes;
    const unsigned blocks = (unsigned)ceil_div(ws.n, kWalkBlock);
#define ORR_GROUPED(W)                                                                                    \
    case W:                                                                                               \
        k_walk_grouped<W, kDescend><<<blocks, kWalkBlock, 0, s>>>(ws.xs, ws.nodes, ws.prm, ws.vals[0], n, nb, \
                                                                         eps2, theta2, out);              \
        break;
    switch (width) {
        ORR_GROUPED(1)
        ORR_GROUPED(2)
        ORR_GROUPED(4)
        ORR_GROUPED(8)
        ORR_GROUPED(16)
        ORR_GROUPED(32)
        ORR_GROUPED(64)
        default:
            return hipErrorInvalidValue;
    }
#undef ORR_GROUPED
    return hipGetLastError();
}

hipError_t launch_walk_grouped(const Workspace &ws, int width, bool descend, float eps2, float theta2, float *acc,
                               uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                               hipStream_t s) {
    const WalkOut out{acc, visits_own, visits_stepped, n_pp, n_pc};
    if (descend) return launch_walk_grouped_t<true>(ws, width, eps2, theta2, out, s);
    return launch_walk_grouped_t<false>(ws, width, eps2, theta2, out, s);
}

}  // namespace orr
