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
// (tile prefix + prefix inside the tile). A node ending at particle e has
// escape = the first node starting at e or later, which is the scan value at
// e. Then one thread per node finds its end: a leaf ends where the next node
// in preorder begins; an internal node's end is searched in the keys.
//
// Moments bottom-up without device-wide synchronisation: the tree is cut into
// subtrees of at most kCutParticles particles ("cut" nodes: the largest nodes
// that small, whose parent is larger); one workgroup finishes each subtree
// level by level with block barriers, then one workgroup finishes the nodes
// above the cut. Every node sums in the fixed order (leaf: its particles in
// sorted order; internal: its children in octant order), so every bit depends
// only on the tree.
#include "checked.h"
#include "orr_internal.h"
#include "schedule.h"

namespace orr {

namespace {

__device__ __forceinline__ int lcp_digits(uint64_t a, uint64_t b) {
    uint64_t x = a ^ b;
    if (x == 0) return kMaxLevel;
    int h = 63 - __clzll((long long)x);  // highest differing bit, 0..62
    return 20 - h / 3;
}

constexpr int kScanTile = 256;

// Nodes started by particles before x: tile prefix + prefix inside the tile.
__device__ __forceinline__ uint32_t base_at(const uint32_t *__restrict__ tile_pre, const uint32_t *__restrict__ loc,
                                            uint32_t x) {
    return tile_pre[x / kScanTile] + loc[x];
}

// One block of 256 particles i in [256 b, 256 b + 256), i <= n. Writes
// info[i] = first(i) | D(i) << 8, loc[i] = nodes started by the block's
// particles before i, and tile_sum[b] = nodes started by the block. Each
// wave of 64 particles is also one target wave of the coherent walk; it
// writes that wave's cost estimate for the walk schedule: summed leaf depth
// D plus 32 times the levels between its deepest leaf and the smallest cell
// holding all its targets (whole levels of the common prefix of its first
// and last key; bit 63 is always zero). At most 64 * 21 + 32 * 21.
__global__ __launch_bounds__(256) void k_tree_count(const uint64_t *__restrict__ keys, uint32_t n, uint32_t cap,
                                                    uint32_t *__restrict__ info, uint32_t *__restrict__ loc,
                                                    uint32_t *__restrict__ tile_sum,
                                                    uint32_t *__restrict__ wave_cost) {
    __shared__ uint64_t sk[256 + 2 * 256];
    __shared__ signed char sw[2][256 + 256];
    __shared__ uint32_t s_wsum[4];
    const int64_t B = (int64_t)blockIdx.x * 256;
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
        sw[0][t] = v;
    }
    __syncthreads();
    // A particle's leaf depth needs the largest of cap + 1 consecutive window
    // values; maxima over 2^k of them come by doubling (level k: sw[k & 1][t]
    // = max of level-0 values [t, t + 2^k)), and the window is two
    // overlapping ones of the largest width that fits. Fewer LDS reads than
    // a scan of cap + 1 values per particle.
    const int W = (int)cap + 1;
    const int kmax = 31 - __clz(W);
    for (int k = 1; k <= kmax; k++) {
        const int half = 1 << (k - 1), cnt = 256 + (int)cap - (1 << k) + 1;
        const signed char *src = sw[(k - 1) & 1];
        signed char *dst = sw[k & 1];
        for (int t = threadIdx.x; t < cnt; t += 256) dst[t] = max(src[t], src[t + half]);
        __syncthreads();
    }
    const int64_t i = B + threadIdx.x;
    uint32_t nst = 0, depth = 0;
    if (i < (int64_t)n) {
        const signed char *mk = sw[kmax & 1];
        const int m = max((int)mk[threadIdx.x], (int)mk[threadIdx.x + W - (1 << kmax)]);
        const int D = min(m + 1, kMaxLevel);
        const int first = (i == 0) ? 0 : lcp_digits(sk[threadIdx.x + cap - 1], sk[threadIdx.x + cap]) + 1;
        info[i] = (uint32_t)first | ((uint32_t)D << 8);
        nst = D >= first ? (uint32_t)(D - first + 1) : 0u;
        depth = (uint32_t)D;
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    {
        uint32_t sum = depth, deepest = depth;
        for (int o = 32; o > 0; o >>= 1) {
            sum += __shfl_xor(sum, o, 64);
            deepest = max(deepest, (uint32_t)__shfl_xor(deepest, o, 64));
        }
        if (lane == 0 && i < (int64_t)n) {
            const int64_t last = min(i + 63, (int64_t)n - 1);
            const uint64_t klast = last - wbeg < wlen ? sk[last - wbeg] : keys[last];
            const uint64_t x = sk[threadIdx.x + cap] ^ klast;
            const uint32_t enclosing = (x == 0ull ? 63u : (uint32_t)__clzll(x) - 1u) / 3u;
            wave_cost[i >> 6] = sum + 32u * (deepest > enclosing ? deepest - enclosing : 0u);
        }
    }
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
    if (i <= (int64_t)n) loc[i] = woff + inc - nst;
    if (threadIdx.x == 0) tile_sum[blockIdx.x] = tot;
}

// One block: exclusive scan of the tile sums in place; the total is n_nodes.
// Wave w takes a contiguous chunk of the tiles (a multiple of 64 of them):
// its sum, read 64 consecutive sums at a time; the 16 wave sums give each
// chunk's offset; then each wave scans its chunk 64 sums at a time (256
// loaded together), carrying the running total. One block barrier in all.
__global__ __launch_bounds__(1024) void k_tile_scan(uint32_t *__restrict__ tile_sum, uint32_t n_tiles,
                                                    DevParams *__restrict__ prm) {
    __shared__ uint32_t s_wsum[16];
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint32_t chunk = ((n_tiles + 15u) / 16u + 63u) / 64u * 64u;
    const uint32_t b = min(w * chunk, n_tiles), e = min(b + chunk, n_tiles);
    uint32_t part = 0;
#pragma unroll 4
    for (uint32_t k = b + lane; k < e; k += 64u) part += tile_sum[k];
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0u) s_wsum[w] = part;
    __syncthreads();
    uint32_t carry = 0, tot = 0;
    for (uint32_t q = 0; q < 16u; q++) {
        if (q < w) carry += s_wsum[q];
        tot += s_wsum[q];
    }
    for (uint32_t k0 = b; k0 < e; k0 += 4u * 64u) {  // four groups of 64 sums loaded together
        uint32_t v[4];
#pragma unroll
        for (uint32_t g = 0; g < 4u; g++) {
            const uint32_t k = k0 + 64u * g + lane;
            v[g] = k < e ? tile_sum[k] : 0u;
        }
#pragma unroll
        for (uint32_t g = 0; g < 4u; g++) {
            const uint32_t k = k0 + 64u * g + lane;
            uint32_t inc = v[g];
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = __shfl_up(inc, o, 64);
                if (lane >= (uint32_t)o) inc += t;
            }
            if (k < e) tile_sum[k] = carry + inc - v[g];
            carry += __shfl(inc, 63, 64);
        }
    }
    if (threadIdx.x == 0) prm->n_nodes = tot;
}

// First j > start whose key differs from pre in its top bits (key >> sh), or
// n; key[start] >> sh == pre. The probes of each round are loaded together,
// eight at a time (offsets 1, 2, 4, ... from start to bracket the end, then
// seven evenly spaced points of the bracket), so the chain of dependent loads
// is a few rounds long instead of two per halving.
__device__ uint32_t cell_end(const uint64_t *__restrict__ keys, uint32_t n, uint32_t start, int sh, uint64_t pre) {
    uint64_t lo = start, hi = n;  // key[lo] in the cell; hi = n or a key outside it
    for (uint32_t q0 = 0; q0 < 64; q0 += 8) {
        uint64_t k[8];
#pragma unroll
        for (uint32_t u = 0; u < 8; u++) {
            const uint64_t p = (uint64_t)start + (1ull << (q0 + u));
            k[u] = p < n ? keys[p] : 0ull;
        }
        bool bracketed = false;
#pragma unroll
        for (uint32_t u = 0; u < 8; u++) {
            const uint64_t p = (uint64_t)start + (1ull << (q0 + u));
            if (bracketed) continue;
            if (p >= n) {
                hi = n;
                bracketed = true;
            } else if ((k[u] >> sh) != pre) {
                hi = p;
                bracketed = true;
            } else {
                lo = p;
            }
        }
        if (bracketed) break;
    }
    while (hi - lo > 1) {
        const uint64_t step = (hi - lo + 7) / 8;  // probes lo + step, lo + 2 step, ... below hi
        uint64_t k[7];
#pragma unroll
        for (uint32_t t = 0; t < 7; t++) {
            const uint64_t p = lo + step * (t + 1);
            k[t] = p < hi ? keys[p] : 0ull;
        }
        uint64_t nlo = lo, nhi = hi;
        bool done = false;
#pragma unroll
        for (uint32_t t = 0; t < 7; t++) {
            const uint64_t p = lo + step * (t + 1);
            if (done || p >= hi) continue;
            if ((k[t] >> sh) != pre) {
                nhi = p;
                done = true;
            } else {
                nlo = p;
            }
        }
        lo = nlo;
        hi = nhi;
    }
    return (uint32_t)hi;
}

// One thread per particle: the level and first particle of every node it
// starts.
__global__ __launch_bounds__(256) void k_tree_stub(const uint32_t *__restrict__ info,
                                                   const uint32_t *__restrict__ tile_pre,
                                                   const uint32_t *__restrict__ loc, uint32_t n,
                                                   NodeRec *__restrict__ nodes, uint8_t *__restrict__ level,
                                                   uint32_t max_nodes, DevParams *__restrict__ prm) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    const uint32_t inf = info[i];
    const int first = (int)(inf & 0xffu), D = (int)(inf >> 8);
    uint32_t node = base_at(tile_pre, loc, i);
    for (int l = first; l <= D; l++, node++) {
        ORR_IF_CHECKED(if (!checked_lt(node, max_nodes, &prm->bad_input)) break;)
        nodes[node].t.y = i;
        level[node] = (uint8_t)l;
    }
}

// Sums of one node, stored for the parent (S, M) and for the walk (com, M).
__device__ __forceinline__ void store_sums(uint32_t k, float M, float sx, float sy, float sz, uint32_t first,
                                           const float4 *__restrict__ xs, NodeRec *nodes, float4 *msum,
                                           const Check &ck) {
    msum[k] = make_float4(sx, sy, sz, M);
    float4 g;
    if (M > 0.0f) {
        g = make_float4(sx / M, sy / M, sz / M, M);  // correctly rounded divisions
    } else {
        const float4 p = checked_lt(first, ck.n_particles, ck.word) ? xs[first] : float4{};
        g = make_float4(p.x, p.y, p.z, M);
    }
    nodes[k].g = g;
}

// Leaf: its particles in sorted order (loads issued four at a time, the sums
// still one particle after the other).
__device__ __forceinline__ void finish_leaf(uint32_t k, uint32_t first, uint32_t count, const float4 *__restrict__ xs,
                                            NodeRec *nodes, float4 *msum, const Check &ck) {
    float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
    const uint32_t end = first + count;
    for (uint32_t j0 = first; j0 < end; j0 += 4) {
        float4 p[4];
#pragma unroll
        for (uint32_t u = 0; u < 4; u++) p[u] = j0 + u < end ? xs[j0 + u] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (uint32_t u = 0; u < 4; u++) {
            if (j0 + u < end) {
                M += p[u].w;
                sx += p[u].w * p[u].x;
                sy += p[u].w * p[u].y;
                sz += p[u].w * p[u].z;
            }
        }
    }
    store_sums(k, M, sx, sy, sz, first, xs, nodes, msum, ck);
}

// One thread per node: its cell end (searched from its first particle), count,
// escape index and s^2; nodes larger than the cut go to the top list; leaves
// also get their moments.
__global__ __launch_bounds__(256) void k_tree_ends(const uint64_t *__restrict__ keys, uint32_t n,
                                                   const uint32_t *__restrict__ tile_pre,
                                                   const uint32_t *__restrict__ loc, DevParams *__restrict__ prm,
                                                   uint32_t max_nodes, NodeRec *nodes,
                                                   const uint8_t *__restrict__ level, uint32_t *__restrict__ top_list,
                                                   uint32_t max_top, const float4 *__restrict__ xs, float4 *msum) {
    const uint32_t k = blockIdx.x * 256u + threadIdx.x;
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    if (k >= nn) return;
    const Check ck{&prm->bad_input, n};
    ORR_IF_CHECKED(if (!checked_lt(prm->n_nodes, (uint64_t)max_nodes + 1u, ck.word)) return;)
    const int l = level[k];
    const uint32_t i = nodes[k].t.y;
    ORR_IF_CHECKED(if (!checked_lt(i, n, ck.word)) return;)
    // In preorder a node is a leaf iff the next node is not its first child
    // (level not above its own); a leaf's particles end where the next node's
    // begin, and its escape is the next index. Internal nodes search for the
    // end of their cell.
    const bool leaf = k + 1 >= nn || (int)level[k + 1] <= l;
    uint32_t end, esc;
    if (leaf) {
        end = k + 1 < nn ? nodes[k + 1].t.y : n;
        esc = k + 1;
    } else {
        const int sh = 3 * (kMaxLevel - l);
        end = l == 0 ? n : cell_end(keys, n, i, sh, keys[i] >> sh);
        esc = base_at(tile_pre, loc, end);
    }
    // a node's particles [i, end) are not empty and lie among the n; its
    // escape is a node index or the end of the tree
    ORR_IF_CHECKED(if (!(checked_lt(i, end, ck.word) && checked_lt(end, (uint64_t)n + 1u, ck.word) &&
                         checked_lt(esc, (uint64_t)nn + 1u, ck.word))) return;)
    const uint32_t count = end - i;
    const float s = ldexpf(prm->side, -l);  // exact
    const float s2 = s * s;
    // begin (t.y) was stored by k_tree_stub and is read here by the previous
    // node's thread (a leaf's end): store only the fields computed here.
    // every record's escape lies beyond its own index (true of any tree, and
    // enforced here whatever the keys): the coherent walk moves to it without
    // a check of its own and still always ends
    nodes[k].t.x = max(esc, k + 1);
    *reinterpret_cast<uint2 *>(&nodes[k].t.z) = make_uint2(count, __float_as_uint(s2));
    if (count > kCutParticles) {
        const uint32_t e = atomicAdd(&prm->n_top, 1u);
        if (checked_lt(e, max_top, ck.word)) top_list[e] = k;
    }
    if (esc == k + 1) finish_leaf(k, i, count, xs, nodes, msum, ck);
}

// Cut nodes (count <= kCutParticles, parent larger or none): the root if no
// node is larger than the cut, else the small children of the nodes above
// the cut. Each of those records its children: kids[9e] = how many,
// kids[9e + 1 ..] = their indices in octant order.
__global__ __launch_bounds__(256) void k_tree_cut(const NodeRec *__restrict__ nodes, DevParams *__restrict__ prm,
                                                  uint32_t max_nodes, const uint32_t *__restrict__ top_list,
                                                  uint32_t max_top, uint32_t *__restrict__ kids,
                                                  uint32_t *__restrict__ cut_list) {
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    const uint32_t n_top = prm->n_top;
    if (n_top == 0) {
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            cut_list[0] = 0;
            prm->n_cut = 1;
        }
        return;
    }
    for (uint32_t e = blockIdx.x * 256u + threadIdx.x; e < n_top; e += gridDim.x * 256u) {
        ORR_IF_CHECKED(if (!checked_lt(e, max_top, &prm->bad_input)) break;)
        const uint32_t k = top_list[e];
        ORR_IF_CHECKED(if (!checked_lt(k, nn, &prm->bad_input)) continue;)
        const uint32_t end = min(nodes[k].t.x, nn);
        uint32_t nk = 0;
        for (uint32_t q = k + 1; q < end && nk < 8;) {
            const uint4 tq = nodes[q].t;
            kids[9 * e + 1 + nk++] = q;
            if (tq.z <= kCutParticles) {
                const uint32_t c = atomicAdd(&prm->n_cut, 1u);
                if (checked_lt(c, max_nodes, &prm->bad_input)) cut_list[c] = q;
            }
            q = max(tq.x, q + 1);
        }
        kids[9 * e] = nk;
    }
}

// Internal node: its children in octant order, by the escape chain.
__device__ __forceinline__ void finish_internal(uint32_t k, const uint4 &t, const float4 *__restrict__ xs,
                                                NodeRec *nodes, float4 *msum, const Check &ck) {
    float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
    for (uint32_t q = k + 1; q < t.x; q = max(nodes[q].t.x, q + 1)) {
        const float4 cs = msum[q];
        M += cs.w;
        sx += cs.x;
        sy += cs.y;
        sz += cs.z;
    }
    store_sums(k, M, sx, sy, sz, t.y, xs, nodes, msum, ck);
}

// Sums of internal node k from its children's, in octant order (escape
// chain), in LDS: esc and sum are indexed from the subtree root.
__device__ __forceinline__ float4 sum_children_lds(uint32_t k, const uint32_t *esc, const float4 *sum) {
    float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
    for (uint32_t q = k + 1; q < esc[k]; q = max(esc[q], q + 1)) {
        const float4 cs = sum[q];
        M += cs.w;
        sx += cs.x;
        sy += cs.y;
        sz += cs.z;
    }
    return make_float4(sx, sy, sz, M);
}

// One workgroup per cut subtree (grid-stride over the cut list): the internal
// nodes of [r, escape(r)) level by level, deepest first (leaves are done).
// A subtree of at most kCutLdsNodes nodes is staged in LDS (escapes, levels,
// sums) and reduced there; a larger one is reduced in global memory.
constexpr uint32_t kCutLdsNodes = 2048;

__global__ __launch_bounds__(256) void k_moments_cut(const float4 *__restrict__ xs, NodeRec *nodes,
                                                     const uint8_t *__restrict__ level,
                                                     const uint32_t *__restrict__ cut_list,
                                                     const DevParams *__restrict__ prm, uint32_t max_nodes,
                                                     float4 *msum) {
    const Check ck = make_check(prm);
    __shared__ float4 s_sum[kCutLdsNodes];
    __shared__ uint32_t s_esc[kCutLdsNodes];
    __shared__ uint8_t s_lvl[kCutLdsNodes];
    __shared__ int s_lmax;
    const uint32_t n_cut = prm->n_cut;
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    for (uint32_t e = blockIdx.x; e < n_cut; e += gridDim.x) {
        // e and r are the same in the whole work-group: the checks below
        // leave its barriers in uniform control flow
        ORR_IF_CHECKED(if (!checked_lt(e, max_nodes, ck.word)) break;)
        const uint32_t r = __builtin_amdgcn_readfirstlane(cut_list[e]);
        ORR_IF_CHECKED(if (!checked_lt(r, nn, ck.word)) continue;)
        const uint32_t end = min(max(nodes[r].t.x, r + 1), nn);
        const uint32_t m = end - r;
        const int lmin = level[r];
        if (threadIdx.x == 0) s_lmax = lmin;
        __syncthreads();  // also: the previous subtree is done with LDS
        int lm = lmin;
        if (m <= kCutLdsNodes) {
            for (uint32_t k = threadIdx.x; k < m; k += 256) {
                const uint32_t ek = min(max(nodes[r + k].t.x, r + k + 1), end) - r;  // stays inside the subtree
                const int l = level[r + k];
                s_esc[k] = ek;
                s_lvl[k] = (uint8_t)l;
                lm = max(lm, l);
                if (ek == k + 1) s_sum[k] = msum[r + k];  // leaf: summed at build
            }
        } else {
            for (uint32_t k = r + threadIdx.x; k < end; k += 256) lm = max(lm, (int)level[k]);
        }
        atomicMax(&s_lmax, lm);
        __syncthreads();
        const int lmax = s_lmax;
        if (m <= kCutLdsNodes) {
            for (int l = lmax; l >= lmin; l--) {
                for (uint32_t k = threadIdx.x; k < m; k += 256)
                    if (s_lvl[k] == l && s_esc[k] != k + 1) s_sum[k] = sum_children_lds(k, s_esc, s_sum);
                __syncthreads();
            }
            for (uint32_t k = threadIdx.x; k < m; k += 256) {
                if (s_esc[k] == k + 1) continue;
                const float4 c = s_sum[k];
                store_sums(r + k, c.w, c.x, c.y, c.z, nodes[r + k].t.y, xs, nodes, msum, ck);
            }
        } else {
            for (int l = lmax; l >= lmin; l--) {
                for (uint32_t k = r + threadIdx.x; k < end; k += 256) {
                    if (level[k] != l) continue;
                    const uint4 t = nodes[k].t;
                    if (t.x != k + 1 && checked_lt(t.x, (uint64_t)nn + 1u, ck.word)) finish_internal(k, t, xs, nodes, msum, ck);
                }
                __syncthreads();
            }
        }
    }
}

// One workgroup: the internal nodes above the cut, level by level, deepest
// first, their children read from the recorded lists. The first
// kTopCached * 1024 entries keep their node, level and children in
// registers; any further ones are read again at every level.
constexpr int kTopCached = 4;

__device__ __forceinline__ void finish_top(uint32_t k, uint32_t nk, const uint32_t *kid,
                                           const float4 *__restrict__ xs, NodeRec *nodes, float4 *msum,
                                           uint32_t nn, const Check &ck) {
    float4 cs[8];
#pragma unroll
    for (uint32_t j = 0; j < 8; j++)
        if (j < nk) cs[j] = checked_lt(kid[j], nn, ck.word) ? msum[kid[j]] : float4{};
    float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
#pragma unroll
    for (uint32_t j = 0; j < 8; j++) {
        if (j >= nk) break;
        M += cs[j].w;
        sx += cs[j].x;
        sy += cs[j].y;
        sz += cs[j].z;
    }
    store_sums(k, M, sx, sy, sz, nodes[k].t.y, xs, nodes, msum, ck);
}

// k_moments_top: block 0 finishes the moments above the cut; blocks 1..8
// build the coherent walk's 8 target-wave lists (schedule.h), independent
// work that runs beside it instead of in a launch of its own.
static_assert(kWaveOrderThreads == 1024, "the schedule blocks have the moments block's size");

__global__ __launch_bounds__(1024) void k_moments_top(const float4 *__restrict__ xs, NodeRec *nodes,
                                                      const uint8_t *__restrict__ level,
                                                      const uint32_t *__restrict__ top_list,
                                                      const uint32_t *__restrict__ kids,
                                                      const DevParams *__restrict__ prm, uint32_t max_nodes,
                                                      uint32_t max_top, float4 *msum,
                                                      const uint32_t *__restrict__ wave_cost, uint32_t n_waves,
                                                      uint32_t *__restrict__ wave_order) {
    if (blockIdx.x >= 1) {
        wave_order_list(wave_cost, n_waves, wave_order, blockIdx.x - 1u);
        return;
    }
    __shared__ int s_lmin, s_lmax;
    const Check chk = make_check(prm);
    const uint32_t nn = min(prm->n_nodes, max_nodes);
    // entries of the list (more than it holds only in a corrupt build, which
    // the checked build reports and clamps)
    const uint32_t n_top = checked_lt(prm->n_top, (uint64_t)max_top + 1u, chk.word) ? prm->n_top : max_top;
    if (threadIdx.x == 0) {
        s_lmin = kMaxLevel + 1;
        s_lmax = -1;
    }
    uint32_t ck[kTopCached], cnk[kTopCached], ckid[kTopCached][8];
    int cl[kTopCached];
#pragma unroll
    for (int j = 0; j < kTopCached; j++) {
        const uint32_t e = threadIdx.x + 1024u * j;
        ck[j] = e < n_top ? top_list[e] : 0u;
        cnk[j] = e < n_top ? kids[9 * e] : 0u;
#pragma unroll
        for (int q = 0; q < 8; q++) ckid[j][q] = e < n_top ? kids[9 * e + 1 + q] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kTopCached; j++)
        cl[j] = threadIdx.x + 1024u * j < n_top && checked_lt(ck[j], nn, chk.word) ? (int)level[ck[j]] : -1;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTopCached; j++)
        if (cl[j] >= 0) {
            atomicMin(&s_lmin, cl[j]);
            atomicMax(&s_lmax, cl[j]);
        }
    for (uint32_t e = threadIdx.x + 1024u * kTopCached; e < n_top; e += 1024) {
        const uint32_t k = top_list[e];
        ORR_IF_CHECKED(if (!checked_lt(k, nn, chk.word)) continue;)
        const int l = level[k];
        atomicMin(&s_lmin, l);
        atomicMax(&s_lmax, l);
    }
    __syncthreads();
    for (int l = s_lmax; l >= s_lmin; l--) {
#pragma unroll
        for (int j = 0; j < kTopCached; j++)
            if (cl[j] == l && cnk[j] != 0) finish_top(ck[j], cnk[j], ckid[j], xs, nodes, msum, nn, chk);
        for (uint32_t e = threadIdx.x + 1024u * kTopCached; e < n_top; e += 1024) {
            const uint32_t k = top_list[e];
            const uint32_t nk = kids[9 * e];
            if (!checked_lt(k, nn, chk.word) || level[k] != l || nk == 0) continue;  // other level, or a leaf (done)
            uint32_t kid[8];
            for (uint32_t q = 0; q < 8; q++) kid[q] = q < nk ? kids[9 * e + 1 + q] : 0u;
            finish_top(k, nk, kid, xs, nodes, msum, nn, chk);
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
    const uint32_t scan_tiles = (uint32_t)ceil_div(ws.n + 1, kScanTile);
    const unsigned node_blocks = (unsigned)ceil_div(ws.max_nodes, 256);
    k_tree_count<<<scan_tiles, 256, 0, s>>>(ws.keys[0], n, (uint32_t)ws.leaf_cap, ws.info, ws.base, ws.tile_sum,
                                            ws.wave_cost);
    k_tile_scan<<<1, 1024, 0, s>>>(ws.tile_sum, scan_tiles, ws.prm);
    k_tree_stub<<<(unsigned)ceil_div(ws.n, 256), 256, 0, s>>>(ws.info, ws.tile_sum, ws.base, n, ws.nodes, ws.level,
                                                              (uint32_t)ws.max_nodes, ws.prm);
    k_tree_ends<<<node_blocks, 256, 0, s>>>(ws.keys[0], n, ws.tile_sum, ws.base, ws.prm, (uint32_t)ws.max_nodes,
                                            ws.nodes, ws.level, ws.top_list, (uint32_t)ws.max_top, ws.xs, ws.msum);
    k_tree_cut<<<64, 256, 0, s>>>(ws.nodes, ws.prm, (uint32_t)ws.max_nodes, ws.top_list, (uint32_t)ws.max_top,
                                  ws.kids, ws.cut_list);
    return hipGetLastError();
}

hipError_t launch_moments(const Workspace &ws, hipStream_t s) {
    // Far more work-groups than the cut subtrees a tree of n particles usually
    // has (the host does not know their number): each reduces its subtrees
    // level by level with a barrier per level, so subtrees that share a
    // work-group add up, and a work-group past the list exits at once.
    const unsigned blocks = (unsigned)std::min<int64_t>(4096, std::max<int64_t>(1, ceil_div(ws.n, kCutParticles) * 64));
    k_moments_cut<<<blocks, 256, 0, s>>>(ws.xs, ws.nodes, ws.level, ws.cut_list, ws.prm, (uint32_t)ws.max_nodes,
                                         ws.msum);
    k_moments_top<<<9, 1024, 0, s>>>(ws.xs, ws.nodes, ws.level, ws.top_list, ws.kids, ws.prm,
                                     (uint32_t)ws.max_nodes, (uint32_t)ws.max_top, ws.msum, ws.wave_cost,
                                     (uint32_t)ws.n_waves, ws.wave_order);
    return hipGetLastError();
}

// The walk schedule of a range of target waves (the range walk), one block
// per XCD list as in k_moments_top.
__global__ __launch_bounds__(kWaveOrderThreads) void k_range_schedule(const uint32_t *__restrict__ wave_cost,
                                                                      uint32_t n_waves,
                                                                      uint32_t *__restrict__ order) {
    wave_order_list(wave_cost, n_waves, order, blockIdx.x);
}

hipError_t launch_range_schedule(const Workspace &ws, int64_t wave0, int64_t n_waves, hipStream_t s) {
    k_range_schedule<<<8, kWaveOrderThreads, 0, s>>>(ws.wave_cost + wave0, (uint32_t)n_waves, ws.range_order);
    return hipGetLastError();
}

hipError_t launch_tree_info(const Workspace &ws, hipStream_t s) {
    k_info_zero<<<1, 1, 0, s>>>(ws.prm);
    k_info<<<(unsigned)ceil_div(ws.max_nodes, 256), 256, 0, s>>>(ws.nodes, ws.level, (uint32_t)ws.max_nodes, ws.prm);
    return hipGetLastError();
}

}  // namespace orr
