// Octree topology, escape indices and monopole moments, built on the device
// from the sorted Morton keys.
//
// The orrery solver page ("Where the tree comes from") builds the tree on the
// host; on a discrete GPU the build runs here instead, without changing the
// tree (definition in include/orr.h).
//
// Topology without recursion. For sorted particle i:
//   * lcp(a, b) = number of leading octal digits two keys share (21 if equal);
//   * the level-l cell holding i has more than cap particles iff some window
//     of cap + 1 consecutive sorted keys containing i shares l digits, i.e.
//     l <= M(i) = max over windows [s, s + cap] with s <= i <= s + cap of
//     lcp(key[s], key[s + cap]) (-1 if no window fits);
//   * so i lies in nodes of levels 0..D(i), D(i) = min(M(i) + 1, 21), its
//     leaf being at D(i), and it is the first particle of its level-l cell
//     iff l > lcp(key[i - 1], key[i]) (every level for i = 0).
// Particle i therefore starts the nodes of levels first(i)..D(i). Depth-first
// preorder is the order of (begin, level), so the node index of (i, l) is
// (nodes started by particles before i) + (l - first(i)), an exclusive scan.
// A node ending at particle e has escape = the first node starting at e or
// later, which is the scan value at e.
//
// Moments bottom-up without level-by-level launches: every leaf sums its
// particles in sorted order, then the last child to finish a parent (counted
// with a device-scope atomic) sums that parent's children in octant order and
// goes on up. The summation order, hence every bit, depends only on the tree.
#include "orr_internal.h"

namespace orr {

namespace {

__device__ __forceinline__ int lcp_digits(uint64_t a, uint64_t b) {
    uint64_t x = a ^ b;
    if (x == 0) return kMaxLevel;
    int h = 63 - __clzll((long long)x);  // highest differing bit, 0..62
    return 20 - h / 3;
}

// One block of 256 particles. Writes info[i] = first(i) | D(i) << 8 and
// nstart[i] = number of nodes i starts; nstart[n] = 0.
__global__ __launch_bounds__(256) void k_tree_count(const uint64_t *__restrict__ keys, uint32_t n, uint32_t cap,
                                                    uint32_t *__restrict__ info, uint32_t *__restrict__ nstart) {
    __shared__ uint64_t sk[256 + 2 * 256];
    __shared__ signed char sw[256 + 256];
    const int64_t B = (int64_t)blockIdx.x * 256;
    const int64_t wbeg = B - (int64_t)cap;
    const int wlen = 256 + 2 * (int)cap;
    for (int t = threadIdx.x; t < wlen; t += 256) {
        int64_t g = wbeg + t;
        sk[t] = (g >= 0 && g < (int64_t)n) ? keys[g] : 0ull;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 256 + (int)cap; t += 256) {
        int64_t s = wbeg + t;
        signed char v = -1;
        if (s >= 0 && s + (int64_t)cap < (int64_t)n) v = (signed char)lcp_digits(sk[t], sk[t + cap]);
        sw[t] = v;
    }
    __syncthreads();
    const int64_t i = B + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x == 0) nstart[n] = 0;
    if (i >= (int64_t)n) return;
    int m = -1;
    for (int t = threadIdx.x; t <= threadIdx.x + (int)cap; t++) m = max(m, (int)sw[t]);
    const int D = min(m + 1, kMaxLevel);
    const int first = (i == 0) ? 0 : lcp_digits(sk[threadIdx.x + cap - 1], sk[threadIdx.x + cap]) + 1;
    info[i] = (uint32_t)first | ((uint32_t)D << 8);
    nstart[i] = D >= first ? (uint32_t)(D - first + 1) : 0u;
}

// First j > i whose key differs from key[i] in its top bits (key >> sh), or n.
__device__ uint32_t cell_end(const uint64_t *__restrict__ keys, uint32_t n, uint32_t i, int sh, uint64_t pre) {
    uint64_t lo = i, hi, step = 1;
    for (;;) {
        uint64_t probe = lo + step;
        if (probe >= n) {
            hi = n;
            break;
        }
        if ((keys[probe] >> sh) != pre) {
            hi = probe;
            break;
        }
        lo = probe;
        step <<= 1;
    }
    while (hi - lo > 1) {
        uint64_t mid = lo + (hi - lo) / 2;
        if ((keys[mid] >> sh) == pre)
            lo = mid;
        else
            hi = mid;
    }
    return (uint32_t)hi;
}

// First j <= i whose key shares key[i]'s top bits (key >> sh).
__device__ uint32_t cell_begin(const uint64_t *__restrict__ keys, uint32_t i, int sh, uint64_t pre) {
    int64_t hi = i, lo, step = 1;
    for (;;) {
        int64_t probe = hi - step;
        if (probe < 0) {
            lo = -1;
            break;
        }
        if ((keys[probe] >> sh) != pre) {
            lo = probe;
            break;
        }
        hi = probe;
        step <<= 1;
    }
    while (hi - lo > 1) {
        int64_t mid = lo + (hi - lo) / 2;
        if ((keys[mid] >> sh) == pre)
            hi = mid;
        else
            lo = mid;
    }
    return (uint32_t)hi;
}

// One thread per particle: write every node the particle starts.
__global__ __launch_bounds__(256) void k_tree_emit(const uint64_t *__restrict__ keys,
                                                   const uint32_t *__restrict__ info,
                                                   const uint32_t *__restrict__ base, uint32_t n,
                                                   const DevParams *__restrict__ prm, NodeRec *__restrict__ nodes,
                                                   uint8_t *__restrict__ level, uint32_t *__restrict__ parent,
                                                   uint32_t *__restrict__ arrive) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    const uint32_t inf = info[i];
    const int first = (int)(inf & 0xffu), D = (int)(inf >> 8);
    if (D < first) return;
    const uint64_t ki = keys[i];
    const float side = prm->side;
    uint32_t node = base[i];
    for (int l = first; l <= D; l++, node++) {
        const int sh = 3 * (kMaxLevel - l);  // 63 at the root: every key maps to 0
        const uint32_t end = cell_end(keys, n, i, sh, ki >> sh);
        const float s = ldexpf(side, -l);  // exact
        const float s2 = s * s;
        nodes[node].t = make_uint4(base[end], i, end - i, __float_as_uint(s2));
        level[node] = (uint8_t)l;
        arrive[node] = 0u;
        uint32_t par;
        if (l == 0) {
            par = kNoParent;
        } else if (l > first) {
            par = node - 1;  // the parent starts at i too
        } else {
            const int shp = 3 * (kMaxLevel - (l - 1));
            const uint32_t b = cell_begin(keys, i, shp, ki >> shp);
            par = base[b] + (uint32_t)(l - 1 - (int)(info[b] & 0xffu));
        }
        parent[node] = par;
    }
}

__device__ __forceinline__ void store_node(uint32_t k, float M, float sx, float sy, float sz, float4 first,
                                           float4 *__restrict__ msum, NodeRec *__restrict__ nodes) {
    msum[k] = make_float4(sx, sy, sz, M);
    float4 g;
    if (M > 0.0f) {
        g = make_float4(sx / M, sy / M, sz / M, M);  // correctly rounded divisions
    } else {
        g = make_float4(first.x, first.y, first.z, M);
    }
    nodes[k].g = g;
}

// One thread per node slot; leaves start, the last child of each parent
// finishes it. No thread waits on another.
__global__ __launch_bounds__(256) void k_moments(const float4 *__restrict__ xs, NodeRec *nodes,
                                                 const uint32_t *__restrict__ parent,
                                                 const DevParams *__restrict__ prm, uint32_t max_nodes,
                                                 float4 *msum, uint32_t *arrive) {
    const uint32_t k = blockIdx.x * 256u + threadIdx.x;
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    if (k >= nn) return;
    const uint4 t = nodes[k].t;
    if (t.x != k + 1) return;  // internal node: finished by its last child
    float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
    for (uint32_t j = t.y; j < t.y + t.z; j++) {
        const float4 p = xs[j];
        M += p.w;
        sx += p.w * p.x;
        sy += p.w * p.y;
        sz += p.w * p.z;
    }
    store_node(k, M, sx, sy, sz, xs[t.y], msum, nodes);
    uint32_t c = k;
    while (c != 0) {
        const uint32_t p = parent[c];
        if (p >= c) return;  // parents precede children in preorder
        const uint4 tp = nodes[p].t;
        uint32_t nch = 0;
        const uint32_t pend = min(tp.x, nn);
        for (uint32_t q = p + 1; q < pend; q = max(nodes[q].t.x, q + 1)) nch++;
        // release this node's sums, then count it; the last arrival acquires
        // every sibling's sums
        const uint32_t old = __hip_atomic_fetch_add(&arrive[p], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old != nch - 1) return;
        M = sx = sy = sz = 0.0f;
        for (uint32_t q = p + 1; q < pend; q = max(nodes[q].t.x, q + 1)) {
            const float4 cs = msum[q];
            M += cs.w;
            sx += cs.x;
            sy += cs.y;
            sz += cs.z;
        }
        store_node(p, M, sx, sy, sz, xs[tp.y], msum, nodes);
        c = p;
    }
}

// Tree statistics for orr_tree_info_get.
__global__ void k_info_zero(DevParams *prm) {
    prm->n_leaves = 0;
    prm->depth = 0;
    prm->max_leaf_count = 0;
}

__global__ __launch_bounds__(256) void k_info(const NodeRec *__restrict__ nodes, const uint8_t *__restrict__ level,
                                              uint32_t max_nodes, DevParams *prm) {
    const uint32_t k = blockIdx.x * 256u + threadIdx.x;
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    uint32_t leaf = 0, dep = 0, cnt = 0;
    if (k < nn) {
        const uint4 t = nodes[k].t;
        dep = level[k];
        if (t.x == k + 1) {
            leaf = 1;
            cnt = t.z;
        }
    }
    // wave-level reduction, then one atomic per wave
    for (int o = 32; o > 0; o >>= 1) {
        leaf += __shfl_xor(leaf, o, 64);
        dep = max(dep, (uint32_t)__shfl_xor(dep, o, 64));
        cnt = max(cnt, (uint32_t)__shfl_xor(cnt, o, 64));
    }
    if ((threadIdx.x & 63) == 0 && leaf) {
        atomicAdd(&prm->n_leaves, leaf);
        atomicMax(&prm->depth, dep);
        atomicMax(&prm->max_leaf_count, cnt);
    }
}

}  // namespace

hipError_t launch_build(const Workspace &ws, hipStream_t s) {
    const uint32_t n = (uint32_t)ws.n;
    const unsigned blocks = (unsigned)ceil_div(ws.n, 256);
    k_tree_count<<<blocks, 256, 0, s>>>(ws.keys[0], n, (uint32_t)ws.leaf_cap, ws.info, ws.base);
    hipError_t e = launch_exclusive_scan(ws.base, ws.base, ws.n + 1, ws.scan_part, &ws.prm->n_nodes, s);
    if (e != hipSuccess) return e;
    k_tree_emit<<<blocks, 256, 0, s>>>(ws.keys[0], ws.info, ws.base, n, ws.prm, ws.nodes, ws.level, ws.parent,
                                       ws.arrive);
    return hipGetLastError();
}

hipError_t launch_moments(const Workspace &ws, hipStream_t s) {
    k_moments<<<(unsigned)ceil_div(ws.max_nodes, 256), 256, 0, s>>>(ws.xs, ws.nodes, ws.parent, ws.prm,
                                                                      (uint32_t)ws.max_nodes, ws.msum, ws.arrive);
    return hipGetLastError();
}

hipError_t launch_tree_info(const Workspace &ws, hipStream_t s) {
    k_info_zero<<<1, 1, 0, s>>>(ws.prm);
    k_info<<<(unsigned)ceil_div(ws.max_nodes, 256), 256, 0, s>>>(ws.nodes, ws.level, (uint32_t)ws.max_nodes, ws.prm);
    return hipGetLastError();
}

}  // namespace orr
