// The two tree walks (enum TreeTraversal of the orrery solver page).
//
// Coherent walk (solver page, "The mitigation"; ADR-0029, Decision): one
// 64-lane wave walks one node index kept in a scalar register. Every lane
// keeps `next`, the node its own walk wants; lanes with next == c act at c,
// the others wait. The wave moves to the smallest `next` of its lanes, which
// is c + 1 if an acting lane opened an internal node and escape[c] otherwise
// (a lane waiting at c skipped an ancestor of c, so its next is at least
// escape[c]); that is one ballot per node. Node records are wave-uniform and
// come through scalar loads; leaf particles are wave-uniform too, so a leaf
// is streamed once for all its opening lanes.
//
// Independent walk (enum TreeTraversal, kIndependent): one lane per target,
// each following its own node index with per-lane vector loads; the measured
// baseline.
//
// Both add the same terms in the same order with the same float operations,
// so their accelerations are identical bit for bit and their visits_own,
// n_pp and n_pc equal the oracle's. Lane i handles sorted target i; outputs
// go straight to the caller's order through perm (the scatter step of the
// performance page's "Where one evaluation goes" table).
#include "orr_internal.h"

namespace orr {

namespace {

// a += m * d * (|d|^2 + eps^2)^(-3/2), every step one correctly rounded float
// operation; the library is compiled without contraction.
__device__ __forceinline__ void add_term(float m, float dx, float dy, float dz, float eps2, float &ax, float &ay,
                                         float &az) {
    const float r2 = ((dx * dx + dy * dy) + dz * dz) + eps2;
    const float inv = 1.0f / sqrtf(r2);
    const float f = m * ((inv * inv) * inv);
    ax += f * dx;
    ay += f * dy;
    az += f * dz;
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

__global__ __launch_bounds__(256) void k_walk_coherent(const float4 *__restrict__ xs,
                                                       const float4 *__restrict__ geom,
                                                       const uint4 *__restrict__ topo,
                                                       const DevParams *__restrict__ prm,
                                                       const uint32_t *__restrict__ perm, uint32_t n,
                                                       uint32_t max_nodes, float eps2, float theta2, WalkOut out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    const bool valid = i < n;
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const float4 xi = valid ? xs[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    uint32_t next = valid ? 0u : n_nodes;  // lanes without a target never act
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    uint32_t vown = 0, vstep = 0, pp = 0, pc = 0;
    uint32_t c = 0;
    while (c < n_nodes) {
        c = __builtin_amdgcn_readfirstlane(c);
        const float4 g = geom[c];
        uint4 t = topo[c];  // (escape, begin, count, s^2 bits)
        t.x = max(t.x, c + 1);  // a well-formed tree has escape > c; never step back
        const bool active = next == c;
        const float dx = g.x - xi.x, dy = g.y - xi.y, dz = g.z - xi.z;
        const float d2 = (dx * dx + dy * dy) + dz * dz;
        const bool accept = active && (__uint_as_float(t.w) < theta2 * d2);
        const bool open = active && !accept;
        vown += active ? 1u : 0u;
        vstep += valid ? 1u : 0u;
        if (__ballot(accept)) {
            if (accept) {
                add_term(g.w, dx, dy, dz, eps2, ax, ay, az);
                pc += 1;
                next = t.x;
            }
        }
        if (t.x == c + 1) {  // leaf
            if (__ballot(open)) {
                const uint32_t e = t.y + t.z;
                for (uint32_t j = t.y; j < e; j++) {
                    const float4 p = xs[j];
                    if (open) add_term(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
                }
                if (open) {
                    pp += t.z - ((i - t.y) < t.z ? 1u : 0u);
                    next = t.x;
                }
            }
            c = t.x;
        } else {
            if (open) next = c + 1;
            c = __ballot(open) ? c + 1 : t.x;
        }
    }
    if (valid) write_out(out, perm[i], ax, ay, az, vown, vstep, pp, pc);
}

__global__ __launch_bounds__(256) void k_walk_independent(const float4 *__restrict__ xs,
                                                          const float4 *__restrict__ geom,
                                                          const uint4 *__restrict__ topo,
                                                          const DevParams *__restrict__ prm,
                                                          const uint32_t *__restrict__ perm, uint32_t n,
                                                          uint32_t max_nodes, float eps2, float theta2,
                                                          WalkOut out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    const uint32_t n_nodes = min(prm->n_nodes, max_nodes);
    const float4 xi = xs[i];
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    uint32_t vown = 0, pp = 0, pc = 0;
    uint32_t c = 0;
    while (c < n_nodes) {
        const float4 g = geom[c];
        uint4 t = topo[c];
        t.x = max(t.x, c + 1);  // a well-formed tree has escape > c; never step back
        const float dx = g.x - xi.x, dy = g.y - xi.y, dz = g.z - xi.z;
        const float d2 = (dx * dx + dy * dy) + dz * dz;
        vown += 1;
        if (__uint_as_float(t.w) < theta2 * d2) {
            add_term(g.w, dx, dy, dz, eps2, ax, ay, az);
            pc += 1;
            c = t.x;
        } else if (t.x == c + 1) {
            const uint32_t e = t.y + t.z;
            for (uint32_t j = t.y; j < e; j++) {
                const float4 p = xs[j];
                add_term(p.w, p.x - xi.x, p.y - xi.y, p.z - xi.z, eps2, ax, ay, az);
            }
            pp += t.z - ((i - t.y) < t.z ? 1u : 0u);
            c = t.x;
        } else {
            c = c + 1;
        }
    }
    write_out(out, perm[i], ax, ay, az, vown, vown, pp, pc);
}

}  // namespace

hipError_t launch_walk(const Workspace &ws, int coherent, float eps2, float theta2, float *acc,
                       uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                       hipStream_t s) {
    const uint32_t n = (uint32_t)ws.n;
    const WalkOut out{acc, visits_own, visits_stepped, n_pp, n_pc};
    const uint32_t nb = (uint32_t)ws.max_nodes;
    const unsigned blocks = (unsigned)ceil_div(ws.n, 256);
    if (coherent)
        k_walk_coherent<<<blocks, 256, 0, s>>>(ws.xs, ws.geom, ws.topo, ws.prm, ws.vals[0], n, nb, eps2, theta2,
                                               out);
    else
        k_walk_independent<<<blocks, 256, 0, s>>>(ws.xs, ws.geom, ws.topo, ws.prm, ws.vals[0], n, nb, eps2,
                                                  theta2, out);
    return hipGetLastError();
}

}  // namespace orr
