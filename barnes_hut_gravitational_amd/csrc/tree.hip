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
// (nodes started by particles before i) + (l - first(i)), an exclusive scan
// (single pass, decoupled look-back). A node ending at particle e has
// escape = the first node starting at e or later, which is the scan value at e.
//
// Moments bottom-up without device-wide synchronisation: the tree is cut into
// subtrees of at most kCutParticles particles ("cut" nodes: the largest nodes
// that small, whose parent is larger); one workgroup finishes each subtree
// level by level with block barriers, then one workgroup finishes the nodes
// above the cut. Every node sums in the fixed order (leaf: its particles in
// sorted order; internal: its children in octant order), so every bit depends
// only on the tree.
#include "orr_internal.h"

namespace orr {

namespace {

__device__ __forceinline__ int lcp_digits(uint64_t a, uint64_t b) {
    uint64_t x = a ^ b;
    if (x == 0) return kMaxLevel;
    int h = 63 - __clzll((long long)x);  // highest differing bit, 0..62
    return 20 - h / 3;
}

constexpr uint64_t kStAggregate = 1ull << 32;
constexpr uint64_t kStInclusive = 2ull << 32;
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr uint32_t kCutParticles = 4096;

// One block of 256 particles (the block's range comes from a ticket, so that
// the tiles before it are running or done). Writes info[i] = first(i) |
// D(i) << 8 and base[i] = nodes started by particles before i, for
// i in [0, n]; base[n] = n_nodes.
__global__ __launch_bounds__(256) void k_tree_count_scan(const uint64_t *__restrict__ keys, uint32_t n,
                                                         uint32_t cap, uint32_t *__restrict__ info,
                                                         uint32_t *__restrict__ base, uint64_t *lb_words,
                                                         DevParams *prm) {
    __shared__ uint64_t sk[256 + 2 * 256];
    __shared__ signed char sw[256 + 256];
    __shared__ uint32_t s_tile, s_wsum[4], s_excl;
    if (threadIdx.x == 0) s_tile = atomicAdd(&prm->scan_ticket, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const int64_t B = (int64_t)tile * 256;
    const int64_t wbeg = B - (int64_t)cap;
    const int wlen = 256 + 2 * (int)cap;
    for (int t = threadIdx.x; t < wlen; t += 256) {
        const int64_t g = wbeg + t;
        sk[t] = (g >= 0 && g < (int64_t)n) ? keys[g] : 0ull;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 256 + (int)cap; t += 256) {
        const int64_t s = wbeg + t;
        signed char v = -1;
        if (s >= 0 && s + (int64_t)cap < (int64_t)n) v = (signed char)lcp_digits(sk[t], sk[t + cap]);
        sw[t] = v;
    }
    __syncthreads();
    const int64_t i = B + threadIdx.x;
    uint32_t nst = 0;
    if (i < (int64_t)n) {
        int m = -1;
        for (int t = threadIdx.x; t <= threadIdx.x + (int)cap; t++) m = max(m, (int)sw[t]);
        const int D = min(m + 1, kMaxLevel);
        const int first = (i == 0) ? 0 : lcp_digits(sk[threadIdx.x + cap - 1], sk[threadIdx.x + cap]) + 1;
        info[i] = (uint32_t)first | ((uint32_t)D << 8);
        nst = D >= first ? (uint32_t)(D - first + 1) : 0u;
    }
    // block exclusive scan of nst, then the tile prefix by look-back
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc = nst;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_wsum[w] = inc;
    __syncthreads();
    uint32_t woff = 0, tot = 0;
    for (int k = 0; k < 4; k++) {
        if (k < w) woff += s_wsum[k];
        tot += s_wsum[k];
    }
    if (threadIdx.x == 0) {
        uint32_t excl = 0;
        if (tile == 0) {
            __hip_atomic_store(lb_words, kStInclusive | tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_store(lb_words + tile, kStAggregate | tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t spins = 0;
            for (int64_t t = (int64_t)tile - 1; t >= 0;) {
                const uint64_t v = __hip_atomic_load(lb_words + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t st = v & ~0xffffffffull;
                if (st == kStInclusive) {
                    excl += (uint32_t)v;
                    break;
                }
                if (st == kStAggregate) {
                    excl += (uint32_t)v;
                    t--;
                    continue;
                }
                if (++spins > kSpinLimit) {
                    atomicOr(&prm->bad_input, 2u);
                    break;
                }
            }
            __hip_atomic_store(lb_words + tile, kStInclusive | (excl + tot), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        s_excl = excl;
    }
    __syncthreads();
    if (i <= (int64_t)n) base[i] = s_excl + woff + inc - nst;  // base[n] = n_nodes
    if (i == (int64_t)n) prm->n_nodes = s_excl + woff + inc - nst;
}

// First j > start whose key differs from pre in its top bits (key >> sh), or
// n; key[start] >> sh == pre.
__device__ uint32_t cell_end(const uint64_t *__restrict__ keys, uint32_t n, uint32_t start, int sh, uint64_t pre) {
    uint64_t lo = start, hi, step = 1;
    for (;;) {
        const uint64_t probe = lo + step;
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
        const uint64_t mid = lo + (hi - lo) / 2;
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
        const int64_t probe = hi - step;
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
        const int64_t mid = lo + (hi - lo) / 2;
        if ((keys[mid] >> sh) == pre)
            hi = mid;
        else
            lo = mid;
    }
    return (uint32_t)hi;
}

// One thread per particle: write every node the particle starts, deepest
// first so that each cell end is searched from the end of the cell inside it;
// list the cut nodes (count <= kCutParticles, parent larger or none) and the
// nodes above the cut.
__global__ __launch_bounds__(256) void k_tree_emit(const uint64_t *__restrict__ keys,
                                                   const uint32_t *__restrict__ info,
                                                   const uint32_t *__restrict__ base, uint32_t n,
                                                   DevParams *__restrict__ prm, NodeRec *__restrict__ nodes,
                                                   uint8_t *__restrict__ level, uint32_t *__restrict__ cut_list,
                                                   uint32_t *__restrict__ top_list) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    const uint32_t inf = info[i];
    const int first = (int)(inf & 0xffu), D = (int)(inf >> 8);
    if (D < first) return;
    const uint64_t ki = keys[i];
    const float side = prm->side;
    const uint32_t node0 = base[i];
    uint32_t end = i + 1, child_count = 0;
    for (int l = D; l >= first; l--) {
        const int sh = 3 * (kMaxLevel - l);  // 63 at the root: every key maps to 0
        end = cell_end(keys, n, end - 1, sh, ki >> sh);
        const uint32_t node = node0 + (uint32_t)(l - first);
        const uint32_t count = end - i;
        const float s = ldexpf(side, -l);  // exact
        const float s2 = s * s;
        nodes[node].t = make_uint4(base[end], i, count, __float_as_uint(s2));
        level[node] = (uint8_t)l;
        // the child started here (level l + 1) is a cut node iff it is small and this node is not
        if (l < D && child_count <= kCutParticles && count > kCutParticles)
            cut_list[atomicAdd(&prm->n_cut, 1u)] = node + 1;
        if (count > kCutParticles) top_list[atomicAdd(&prm->n_top, 1u)] = node;
        child_count = count;
    }
    // the node of level first: its parent starts before i (or it is the root)
    if (child_count <= kCutParticles) {
        bool cut = first == 0;
        if (first > 0) {
            const int shp = 3 * (kMaxLevel - (first - 1));
            const uint64_t prep = ki >> shp;
            const uint32_t pb = cell_begin(keys, i, shp, prep);
            const uint32_t pe = cell_end(keys, n, end - 1, shp, prep);
            cut = pe - pb > kCutParticles;
        }
        if (cut) cut_list[atomicAdd(&prm->n_cut, 1u)] = node0;
    }
}

__device__ __forceinline__ void finish_node(uint32_t k, const uint4 &t, const float4 *__restrict__ xs,
                                            NodeRec *nodes, float4 *msum) {
    float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
    if (t.x == k + 1) {  // leaf: its particles in sorted order
        for (uint32_t j = t.y; j < t.y + t.z; j++) {
            const float4 p = xs[j];
            M += p.w;
            sx += p.w * p.x;
            sy += p.w * p.y;
            sz += p.w * p.z;
        }
    } else {  // internal: its children in octant order
        for (uint32_t q = k + 1; q < t.x; q = max(nodes[q].t.x, q + 1)) {
            const float4 cs = msum[q];
            M += cs.w;
            sx += cs.x;
            sy += cs.y;
            sz += cs.z;
        }
    }
    msum[k] = make_float4(sx, sy, sz, M);
    float4 g;
    if (M > 0.0f) {
        g = make_float4(sx / M, sy / M, sz / M, M);  // correctly rounded divisions
    } else {
        const float4 p = xs[t.y];
        g = make_float4(p.x, p.y, p.z, M);
    }
    nodes[k].g = g;
}

// One workgroup per cut subtree (grid-stride over the cut list): the nodes of
// [r, escape(r)) level by level, deepest first.
__global__ __launch_bounds__(256) void k_moments_cut(const float4 *__restrict__ xs, NodeRec *nodes,
                                                     const uint8_t *__restrict__ level,
                                                     const uint32_t *__restrict__ cut_list,
                                                     const DevParams *__restrict__ prm, uint32_t max_nodes,
                                                     float4 *msum) {
    __shared__ int s_lmax;
    const uint32_t n_cut = prm->n_cut;
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    for (uint32_t e = blockIdx.x; e < n_cut; e += gridDim.x) {
        const uint32_t r = cut_list[e];
        const uint32_t end = min(max(nodes[r].t.x, r + 1), nn);
        const int lmin = level[r];
        if (threadIdx.x == 0) s_lmax = lmin;
        __syncthreads();
        int lm = lmin;
        for (uint32_t k = r + threadIdx.x; k < end; k += 256) lm = max(lm, (int)level[k]);
        atomicMax(&s_lmax, lm);
        __syncthreads();
        const int lmax = s_lmax;
        for (int l = lmax; l >= lmin; l--) {
            for (uint32_t k = r + threadIdx.x; k < end; k += 256)
                if (level[k] == l) finish_node(k, nodes[k].t, xs, nodes, msum);
            __syncthreads();
        }
    }
}

// One workgroup: the nodes above the cut, level by level, deepest first.
__global__ __launch_bounds__(1024) void k_moments_top(const float4 *__restrict__ xs, NodeRec *nodes,
                                                      const uint8_t *__restrict__ level,
                                                      const uint32_t *__restrict__ top_list,
                                                      const DevParams *__restrict__ prm, float4 *msum) {
    __shared__ int s_lmin, s_lmax;
    const uint32_t n_top = prm->n_top;
    if (threadIdx.x == 0) {
        s_lmin = kMaxLevel + 1;
        s_lmax = -1;
    }
    __syncthreads();
    for (uint32_t e = threadIdx.x; e < n_top; e += 1024) {
        const int l = level[top_list[e]];
        atomicMin(&s_lmin, l);
        atomicMax(&s_lmax, l);
    }
    __syncthreads();
    for (int l = s_lmax; l >= s_lmin; l--) {
        for (uint32_t e = threadIdx.x; e < n_top; e += 1024) {
            const uint32_t k = top_list[e];
            if (level[k] == l) finish_node(k, nodes[k].t, xs, nodes, msum);
        }
        __syncthreads();
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
    k_tree_count_scan<<<(unsigned)ceil_div(ws.n + 1, 256), 256, 0, s>>>(ws.keys[0], n, (uint32_t)ws.leaf_cap, ws.info,
                                                                       ws.base, ws.lb_words + ws.lb_scan_offset,
                                                                       ws.prm);
    k_tree_emit<<<(unsigned)ceil_div(ws.n, 256), 256, 0, s>>>(ws.keys[0], ws.info, ws.base, n, ws.prm, ws.nodes,
                                                              ws.level, ws.cut_list, ws.top_list);
    return hipGetLastError();
}

hipError_t launch_moments(const Workspace &ws, hipStream_t s) {
    const unsigned blocks = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(ws.n, kCutParticles) * 2));
    k_moments_cut<<<blocks, 256, 0, s>>>(ws.xs, ws.nodes, ws.level, ws.cut_list, ws.prm, (uint32_t)ws.max_nodes,
                                         ws.msum);
    k_moments_top<<<1, 1024, 0, s>>>(ws.xs, ws.nodes, ws.level, ws.top_list, ws.prm, ws.msum);
    return hipGetLastError();
}

hipError_t launch_tree_info(const Workspace &ws, hipStream_t s) {
    k_info_zero<<<1, 1, 0, s>>>(ws.prm);
    k_info<<<(unsigned)ceil_div(ws.max_nodes, 256), 256, 0, s>>>(ws.nodes, ws.level, (uint32_t)ws.max_nodes, ws.prm);
    return hipGetLastError();
}

}  // namespace orr
