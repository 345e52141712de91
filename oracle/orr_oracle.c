/*
 * CPU oracle for the Barnes-Hut force evaluation with the masked coherent walk.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path never
 * calls it, and it shares no code, header or table with the HIP library.
 *
 * Plain, slow and single-threaded except for the loops over independent
 * targets (OpenMP). Compiled with -ffp-contract=off and without -ffast-math so
 * that every floating-point step is one IEEE single-precision operation
 * rounded to nearest, in the order written.
 *
 * Sources (the orrery pages):
 *   [SOLVER] "sycl_tree_solver.hpp" page: "The mitigation", "What is not given
 *            up", "Where the tree comes from", enum TreeTraversal.
 *   [ADR29]  "ADR-0029: mask the accepted cells rather than descending
 *            together": Decision, Alternatives considered, Consequences.
 *   [PERF]   "docs/performance/sycl_tree.md": table "The machine and the
 *            device" (Plummer, softening 0.05, opening angle 0.5, leaf
 *            capacity 32, monopole only), "Where one evaluation goes" (Morton
 *            sort, gather, build, node staging, walk, scatter), "Accuracy"
 *            (compensated double-precision direct sum as the reference).
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KEY_BITS_PER_AXIS 21
#define MAX_LEVEL 21
#define Q_MAX 2097151u /* 2^21 - 1 */

enum { ORACLE_OK = 0, ORACLE_INVALID = 1, ORACLE_RANGE = 2, ORACLE_NONFINITE = 3, ORACLE_NOMEM = 5 };

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the later parallel loops (timing only; results do not depend on it). */
void oracle_set_num_threads(int k) {
#ifdef _OPENMP
    if (k >= 1) omp_set_num_threads(k);
#else
    (void)k;
#endif
}

/* ------------------------------------------------------------------------ */
/* Root cell. [PERF] "Where one evaluation goes" names a Morton sort; the    */
/* pages do not say how the root cube is chosen. Reading: a tight cube whose */
/* corner is the component-wise minimum and whose side is the largest        */
/* per-axis extent; a zero extent becomes side 1. The +0.0f turns a -0       */
/* minimum into +0 so that the corner is unique.                             */
/* ------------------------------------------------------------------------ */
int oracle_root_cube(const float *pos, const float *mass, int64_t n, float lo[3], float *side,
                     float *scale) {
    if (n < 1) return ORACLE_RANGE;
    float mn[3], mx[3];
    for (int a = 0; a < 3; a++) mn[a] = mx[a] = pos[a];
    for (int64_t i = 0; i < n; i++) {
        for (int a = 0; a < 3; a++) {
            float x = pos[3 * i + a];
            if (!isfinite(x)) return ORACLE_NONFINITE;
            if (x < mn[a]) mn[a] = x;
            if (x > mx[a]) mx[a] = x;
        }
        if (!isfinite(mass[i]) || mass[i] < 0.0f) return ORACLE_NONFINITE;
    }
    float L = 0.0f;
    for (int a = 0; a < 3; a++) {
        lo[a] = mn[a] + 0.0f;
        float ext = mx[a] - lo[a];
        if (ext > L) L = ext;
    }
    if (!isfinite(L)) return ORACLE_NONFINITE;
    if (L == 0.0f) L = 1.0f;
    *side = L;
    *scale = 2097152.0f / L;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Morton keys ([PERF] "Morton sort"). Reading: 21 bits per axis, each       */
/* coordinate quantised as trunc((x - lo) * scale) with two separately       */
/* rounded float operations and clamped to 2^21 - 1; the 63-bit key holds    */
/* bit b of x, y, z at bits 3b+2, 3b+1, 3b. The octant digit that selects a  */
/* child at level l is therefore (key >> 3(21 - l)) & 7.                     */
/* ------------------------------------------------------------------------ */
static uint32_t quantise(float x, float lo, float scale) {
    float t = (x - lo) * scale;
    if (t >= 2097151.0f) return Q_MAX;
    return (uint32_t)t;
}

uint64_t oracle_interleave(uint32_t qx, uint32_t qy, uint32_t qz) {
    uint64_t key = 0;
    for (int b = 0; b < KEY_BITS_PER_AXIS; b++) {
        key |= (uint64_t)((qx >> b) & 1u) << (3 * b + 2);
        key |= (uint64_t)((qy >> b) & 1u) << (3 * b + 1);
        key |= (uint64_t)((qz >> b) & 1u) << (3 * b);
    }
    return key;
}

void oracle_morton_keys(const float *pos, int64_t n, const float lo[3], float scale, uint64_t *keys) {
    for (int64_t i = 0; i < n; i++) {
        uint32_t qx = quantise(pos[3 * i + 0], lo[0], scale);
        uint32_t qy = quantise(pos[3 * i + 1], lo[1], scale);
        uint32_t qz = quantise(pos[3 * i + 2], lo[2], scale);
        keys[i] = oracle_interleave(qx, qy, qz);
    }
}

/* ------------------------------------------------------------------------ */
/* Sort into tree order. Equal keys keep ascending original index, so the    */
/* order is unique: qsort over (key, index) pairs with a total order.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    uint64_t key;
    uint32_t idx;
} key_idx;

static int cmp_key_idx(const void *pa, const void *pb) {
    const key_idx *a = (const key_idx *)pa, *b = (const key_idx *)pb;
    if (a->key != b->key) return a->key < b->key ? -1 : 1;
    if (a->idx != b->idx) return a->idx < b->idx ? -1 : 1;
    return 0;
}

int oracle_sort(const uint64_t *keys, int64_t n, uint32_t *perm, uint64_t *keys_sorted) {
    key_idx *t = (key_idx *)malloc((size_t)n * sizeof(key_idx));
    if (!t) return ORACLE_NOMEM;
    for (int64_t i = 0; i < n; i++) {
        t[i].key = keys[i];
        t[i].idx = (uint32_t)i;
    }
    qsort(t, (size_t)n, sizeof(key_idx), cmp_key_idx);
    for (int64_t i = 0; i < n; i++) {
        perm[i] = t[i].idx;
        keys_sorted[i] = t[i].key;
    }
    free(t);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Octree ([SOLVER] "Where the tree comes from"; [PERF] leaf capacity 32).   */
/* A node at level l covers a run of sorted keys sharing their top 3l bits.  */
/* It is split iff it holds more than leaf_cap particles and l < 21; its     */
/* children are its non-empty octants in digit order. Nodes are numbered in  */
/* depth-first preorder, so the first child of node k is k + 1, and the      */
/* escape index of k (where a walk goes after accepting k or finishing a     */
/* leaf, [ADR29] Decision) is k plus the size of its subtree.               */
/* ------------------------------------------------------------------------ */
typedef struct {
    const uint64_t *keys;
    int64_t leaf_cap;
    int64_t n_nodes, max_nodes;
    uint8_t *level;
    uint32_t *begin, *count, *escape;
    int overflow;
} builder;

static void build_node(builder *B, int lvl, int64_t b, int64_t e) {
    if (B->n_nodes >= B->max_nodes) {
        B->overflow = 1;
        return;
    }
    int64_t me = B->n_nodes++;
    B->level[me] = (uint8_t)lvl;
    B->begin[me] = (uint32_t)b;
    B->count[me] = (uint32_t)(e - b);
    if (e - b > B->leaf_cap && lvl < MAX_LEVEL) {
        int shift = 3 * (MAX_LEVEL - (lvl + 1));
        int64_t j = b;
        for (uint64_t d = 0; d < 8; d++) {
            int64_t k = j;
            while (k < e && ((B->keys[k] >> shift) & 7u) == d) k++;
            if (k > j) build_node(B, lvl + 1, j, k);
            j = k;
        }
    }
    B->escape[me] = (uint32_t)B->n_nodes;
}

/* Returns the node count, or -1 if max_nodes is too small. */
int64_t oracle_build(const uint64_t *keys_sorted, int64_t n, int32_t leaf_cap, int64_t max_nodes,
                     uint8_t *level, uint32_t *begin, uint32_t *count, uint32_t *escape) {
    builder B = {keys_sorted, leaf_cap, 0, max_nodes, level, begin, count, escape, 0};
    build_node(&B, 0, 0, n);
    return B.overflow ? -1 : B.n_nodes;
}

/* ------------------------------------------------------------------------ */
/* Monopole moments ([PERF] "monopole only"). Reading of the fixed order:    */
/* a leaf sums its particles in sorted order, M += m_j and S += m_j * x_j    */
/* (product rounded, then sum rounded); an internal node sums its children's */
/* M and S in octant order; com = S / M, or the node's first particle when   */
/* M = 0. Children come before parents in reverse preorder. The node side is */
/* side * 2^-level (exact) and s2 = side^2 rounded once.                     */
/* xs holds sorted particles as (x, y, z, m).                                */
/* ------------------------------------------------------------------------ */
int oracle_moments(const float *xs, int64_t n_nodes, const uint8_t *level, const uint32_t *begin,
                   const uint32_t *count, const uint32_t *escape, float side, float *geom, float *s2) {
    float *S = (float *)malloc((size_t)n_nodes * 4 * sizeof(float));
    if (!S) return ORACLE_NOMEM;
    for (int64_t k = n_nodes - 1; k >= 0; k--) {
        float M = 0.0f, sx = 0.0f, sy = 0.0f, sz = 0.0f;
        if (escape[k] == (uint32_t)(k + 1)) {
            for (uint32_t j = begin[k]; j < begin[k] + count[k]; j++) {
                const float *p = xs + 4 * (size_t)j;
                M += p[3];
                sx += p[3] * p[0];
                sy += p[3] * p[1];
                sz += p[3] * p[2];
            }
        } else {
            for (uint32_t c = (uint32_t)k + 1; c < escape[k]; c = escape[c]) {
                M += S[4 * c + 3];
                sx += S[4 * c + 0];
                sy += S[4 * c + 1];
                sz += S[4 * c + 2];
            }
        }
        S[4 * k + 0] = sx;
        S[4 * k + 1] = sy;
        S[4 * k + 2] = sz;
        S[4 * k + 3] = M;
        float *g = geom + 4 * k;
        if (M > 0.0f) {
            g[0] = sx / M;
            g[1] = sy / M;
            g[2] = sz / M;
        } else {
            const float *p = xs + 4 * (size_t)begin[k];
            g[0] = p[0];
            g[1] = p[1];
            g[2] = p[2];
        }
        g[3] = M;
        float s = ldexpf(side, -(int)level[k]);
        s2[k] = s * s;
    }
    free(S);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Softened monopole term ([PERF] softening 0.05; "Accuracy": the same       */
/* softened force law as the reference). G = 1:                              */
/*   a += m d (|d|^2 + eps^2)^(-3/2),  d = source - target.                  */
/* Operation order: r2 = ((dx*dx + dy*dy) + dz*dz) + eps2,                  */
/* inv = 1 / sqrt(r2) (two correctly rounded operations), f = m*((inv*inv)*  */
/* inv), then a_x += f*dx and likewise for y and z.                          */
/* ------------------------------------------------------------------------ */
static void add_term(float m, float dx, float dy, float dz, float eps2, float a[3]) {
    float r2 = ((dx * dx + dy * dy) + dz * dz) + eps2;
    float inv = 1.0f / sqrtf(r2);
    float f = m * ((inv * inv) * inv);
    a[0] += f * dx;
    a[1] += f * dy;
    a[2] += f * dz;
}

/* The target's own term is m * 0 * eps^-3 (d = 0), +0 as the force law     */
/* wants only while eps^-3, evaluated as add_term evaluates it, is finite:   */
/* 1 if so, 0 if eps is not finite and positive or that cube overflows (the  */
/* own term, and so every sum, would be 0 * inf = NaN).                      */
int oracle_eps_ok(float eps) {
    if (!(isfinite(eps) && eps > 0.0f)) return 0;
    float eps2 = eps * eps;
    if (!(eps2 > 0.0f)) return 0;
    float inv = 1.0f / sqrtf(eps2);
    return isfinite((inv * inv) * inv) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* One target's stackless walk ([ADR29] Decision; [SOLVER] "What is not      */
/* given up": each target is summed over exactly the nodes its own walk      */
/* visits, in the same order). Opening test at every node, leaves included:  */
/* accept iff s2 < theta2 * d2 with d = com - x (s/d < theta, strict).       */
/*   accept            -> monopole term, pc += 1, go to escape              */
/*   open, leaf        -> every particle of the leaf in sorted order,        */
/*                        pp += count minus the target itself, go to escape  */
/*   open, internal    -> go to the first child, k + 1                       */
/* The target's own term is evaluated and is +0 (d = 0); it is not counted.  */
/* If trace is non-null it receives (node << 2 | action) per visit, action   */
/* 0 = accepted, 1 = opened leaf, 2 = opened internal node.                  */
/* ------------------------------------------------------------------------ */
typedef struct {
    const float *xs;
    const float *geom;
    const float *s2;
    const uint32_t *begin, *count, *escape;
    int64_t n_nodes;
    float eps2, theta2;
} walk_ctx;

static void walk_one(const walk_ctx *W, int64_t i, float a[3], uint32_t *pp, uint32_t *pc,
                     uint32_t *visits, uint64_t *trace, int64_t trace_cap) {
    const float *xi = W->xs + 4 * (size_t)i;
    a[0] = a[1] = a[2] = 0.0f;
    uint32_t npp = 0, npc = 0, nv = 0;
    int64_t c = 0;
    while (c < W->n_nodes) {
        const float *g = W->geom + 4 * c;
        float dx = g[0] - xi[0], dy = g[1] - xi[1], dz = g[2] - xi[2];
        float d2 = (dx * dx + dy * dy) + dz * dz;
        int action;
        if (W->s2[c] < W->theta2 * d2) {
            add_term(g[3], dx, dy, dz, W->eps2, a);
            npc += 1;
            action = 0;
        } else if (W->escape[c] == (uint32_t)(c + 1)) {
            uint32_t b = W->begin[c], e = W->begin[c] + W->count[c];
            for (uint32_t j = b; j < e; j++) {
                const float *p = W->xs + 4 * (size_t)j;
                add_term(p[3], p[0] - xi[0], p[1] - xi[1], p[2] - xi[2], W->eps2, a);
            }
            npp += W->count[c] - ((i >= b && i < e) ? 1u : 0u);
            action = 1;
        } else {
            action = 2;
        }
        if (trace && nv < trace_cap) trace[nv] = ((uint64_t)c << 2) | (uint64_t)action;
        nv += 1;
        c = (action == 2) ? c + 1 : (int64_t)W->escape[c];
    }
    *pp = npp;
    *pc = npc;
    *visits = nv;
}

/* Walk the sorted targets listed in `targets` (or all n if targets == NULL).
 * Outputs are indexed like `targets` (acc has 3 floats per entry). */
void oracle_walk(const float *xs, int64_t n, const float *geom, const float *s2, const uint32_t *begin,
                 const uint32_t *count, const uint32_t *escape, int64_t n_nodes, float eps, float theta,
                 const int64_t *targets, int64_t n_targets, float *acc, uint32_t *pp, uint32_t *pc,
                 uint32_t *visits) {
    walk_ctx W = {xs, geom, s2, begin, count, escape, n_nodes, eps * eps, theta * theta};
    int64_t m = targets ? n_targets : n;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < m; t++) {
        int64_t i = targets ? targets[t] : t;
        walk_one(&W, i, acc + 3 * t, pp + t, pc + t, visits + t, NULL, 0);
    }
}

/* One target's visit sequence, for tests. Returns the number of visits. */
int64_t oracle_walk_trace(const float *xs, const float *geom, const float *s2, const uint32_t *begin,
                          const uint32_t *count, const uint32_t *escape, int64_t n_nodes, float eps,
                          float theta, int64_t target, uint64_t *trace, int64_t trace_cap) {
    walk_ctx W = {xs, geom, s2, begin, count, escape, n_nodes, eps * eps, theta * theta};
    float a[3];
    uint32_t pp, pc, nv;
    walk_one(&W, target, a, &pp, &pc, &nv, trace, trace_cap);
    return (int64_t)nv;
}

/* ------------------------------------------------------------------------ */
/* Nodes stepped through by a coherent group ([PERF] "The divergence         */
/* mitigation": a coherent lane's visits are its whole group's union,        */
/* counted once per lane; [ADR29] Decision: the group's sequence is exactly  */
/* the union of its lanes' walks). Groups are `width` consecutive sorted     */
/* targets, the last one possibly partial. Plain definition: the size of the */
/* set union of the members' own walks, computed with a bit set.             */
/* out[k] = union size of group group_ids[k] (of group k if group_ids is     */
/* NULL, all groups).                                                        */
/* ------------------------------------------------------------------------ */
int oracle_union_visits(const float *xs, int64_t n, const float *geom, const float *s2,
                        const uint32_t *begin, const uint32_t *count, const uint32_t *escape,
                        int64_t n_nodes, float eps, float theta, int64_t width, const int64_t *group_ids,
                        int64_t n_groups, uint32_t *out) {
    walk_ctx W = {xs, geom, s2, begin, count, escape, n_nodes, eps * eps, theta * theta};
    int64_t groups = group_ids ? n_groups : (n + width - 1) / width;
    int64_t words = (n_nodes + 63) / 64;
    int failed = 0;
#pragma omp parallel
    {
        uint64_t *bits = (uint64_t *)malloc((size_t)words * sizeof(uint64_t));
        uint64_t *trace = (uint64_t *)malloc((size_t)n_nodes * sizeof(uint64_t));
        if (!bits || !trace) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t gi = 0; gi < groups; gi++) {
                int64_t g = group_ids ? group_ids[gi] : gi;
                memset(bits, 0, (size_t)words * sizeof(uint64_t));
                int64_t hi = (g + 1) * width < n ? (g + 1) * width : n;
                for (int64_t i = g * width; i < hi; i++) {
                    float a[3];
                    uint32_t pp, pc, nv;
                    walk_one(&W, i, a, &pp, &pc, &nv, trace, n_nodes);
                    for (uint32_t v = 0; v < nv; v++) {
                        uint64_t node = trace[v] >> 2;
                        bits[node >> 6] |= 1ull << (node & 63);
                    }
                }
                uint32_t total = 0;
                for (int64_t w = 0; w < words; w++) total += (uint32_t)__builtin_popcountll(bits[w]);
                out[gi] = total;
            }
        }
        free(bits);
        free(trace);
    }
    return failed ? ORACLE_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Simulation of the group walk itself, for tests of the advance rule.       */
/* rule 0 ([ADR29] Decision): every lane keeps `next`, the node its own walk */
/* wants; the group node is the minimum over lanes; lanes whose next equals  */
/* it act, the others wait.                                                 */
/* rule 1: the same lanes act, but the group moves to node + 1 if any acting */
/* lane opened an internal node and to the node's escape index otherwise.    */
/* Per group: steps[g] = nodes the group stepped through. Per lane, in       */
/* sorted order: own[i] = nodes where the lane acted. Returns 0, or 1 if the */
/* ballot rule ever stepped to a node no lane wanted.                        */
/* ------------------------------------------------------------------------ */
int oracle_group_walk(const float *xs, int64_t n, const float *geom, const float *s2,
                      const uint32_t *begin, const uint32_t *count, const uint32_t *escape,
                      int64_t n_nodes, float eps, float theta, int64_t width, int rule, uint32_t *steps,
                      uint32_t *own) {
    float eps2 = eps * eps, theta2 = theta * theta;
    (void)eps2;
    (void)begin;
    (void)count;
    int64_t groups = (n + width - 1) / width;
    int bad = 0;
    int64_t *next = (int64_t *)malloc((size_t)width * sizeof(int64_t));
    if (!next) return ORACLE_NOMEM;
    for (int64_t g = 0; g < groups; g++) {
        int64_t lo = g * width, hi = (g + 1) * width < n ? (g + 1) * width : n;
        for (int64_t l = 0; l < width; l++) next[l] = (lo + l < hi) ? 0 : n_nodes;
        for (int64_t i = lo; i < hi; i++) own[i] = 0;
        uint32_t nsteps = 0;
        int64_t c = 0;
        while (c < n_nodes) {
            nsteps += 1;
            int any_active = 0, any_descend = 0;
            for (int64_t l = 0; l < hi - lo; l++) {
                if (next[l] != c) continue;
                any_active = 1;
                own[lo + l] += 1;
                const float *xi = xs + 4 * (size_t)(lo + l);
                const float *gm = geom + 4 * c;
                float dx = gm[0] - xi[0], dy = gm[1] - xi[1], dz = gm[2] - xi[2];
                float d2 = (dx * dx + dy * dy) + dz * dz;
                if (s2[c] < theta2 * d2 || escape[c] == (uint32_t)(c + 1)) {
                    next[l] = escape[c];
                } else {
                    next[l] = c + 1;
                    any_descend = 1;
                }
            }
            if (!any_active) bad = 1;
            if (rule == 0) {
                int64_t m = n_nodes;
                for (int64_t l = 0; l < width; l++)
                    if (next[l] < m) m = next[l];
                c = m;
            } else {
                c = any_descend ? c + 1 : (int64_t)escape[c];
            }
        }
        steps[g] = nsteps;
    }
    free(next);
    return bad;
}

/* ------------------------------------------------------------------------ */
/* The alternative [ADR29] rejects ("Alternatives considered": descend       */
/* wherever any lane must, and let the accepting lanes descend too), which   */
/* is the published warp-coherent traversal. Groups of `width` consecutive   */
/* sorted targets share one node c. Every member applies the opening test at */
/* c. If at least one member would open c, the whole group opens it: at a    */
/* leaf every member adds the leaf's particles in sorted order, and at an    */
/* internal node the group moves to c + 1 without terms. If no member would  */
/* open c, every member adds c's monopole term and the group moves to        */
/* escape[c]. Terms use add_term, in visit order. Per sorted target:         */
/* acc, pp (particle terms, self excluded), pc (accepted cells), visits      */
/* (nodes the group stepped through; the target acts at each), covered       */
/* (particles accounted for: counts of its accepted cells plus the counts of */
/* its opened leaves, which is n when every particle is summed once).        */
/* ------------------------------------------------------------------------ */
int oracle_walk_descend(const float *xs, int64_t n, const float *geom, const float *s2, const uint32_t *begin,
                        const uint32_t *count, const uint32_t *escape, int64_t n_nodes, float eps, float theta,
                        int64_t width, float *acc, uint32_t *pp, uint32_t *pc, uint32_t *visits,
                        uint32_t *covered) {
    const float eps2 = eps * eps, theta2 = theta * theta;
    const int64_t groups = (n + width - 1) / width;
    int failed = 0;
#pragma omp parallel
    {
        float *d = (float *)malloc((size_t)width * 4 * sizeof(float));
        if (!d) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t g = 0; g < groups; g++) {
                const int64_t lo = g * width, hi = (g + 1) * width < n ? (g + 1) * width : n;
                for (int64_t i = lo; i < hi; i++) {
                    acc[3 * i] = acc[3 * i + 1] = acc[3 * i + 2] = 0.0f;
                    pp[i] = pc[i] = visits[i] = covered[i] = 0;
                }
                int64_t c = 0;
                while (c < n_nodes) {
                    const float *gm = geom + 4 * c;
                    int any_open = 0;
                    for (int64_t i = lo; i < hi; i++) {
                        const float *xi = xs + 4 * (size_t)i;
                        float *di = d + 4 * (i - lo);
                        di[0] = gm[0] - xi[0];
                        di[1] = gm[1] - xi[1];
                        di[2] = gm[2] - xi[2];
                        di[3] = (di[0] * di[0] + di[1] * di[1]) + di[2] * di[2];
                        if (!(s2[c] < theta2 * di[3])) any_open = 1;
                        visits[i] += 1;
                    }
                    if (any_open) {
                        if (escape[c] == (uint32_t)(c + 1)) {
                            const uint32_t b = begin[c], e = begin[c] + count[c];
                            for (int64_t i = lo; i < hi; i++) {
                                const float *xi = xs + 4 * (size_t)i;
                                for (uint32_t j = b; j < e; j++) {
                                    const float *p = xs + 4 * (size_t)j;
                                    add_term(p[3], p[0] - xi[0], p[1] - xi[1], p[2] - xi[2], eps2, acc + 3 * i);
                                }
                                pp[i] += count[c] - ((i >= b && i < e) ? 1u : 0u);
                                covered[i] += count[c];
                            }
                        }
                        c = c + 1;
                    } else {
                        for (int64_t i = lo; i < hi; i++) {
                            const float *di = d + 4 * (i - lo);
                            add_term(gm[3], di[0], di[1], di[2], eps2, acc + 3 * i);
                            pc[i] += 1;
                            covered[i] += count[c];
                        }
                        c = (int64_t)escape[c];
                    }
                }
            }
        }
        free(d);
    }
    return failed ? ORACLE_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Float32 direct sum, the all-pairs reference (the direct solver of the     */
/* orrery pages, "Against the two solvers it has to beat"): for each listed  */
/* caller-order target i, a_i = sum over every particle j in index order of  */
/* the same softened term as the walk's (add_term), the target's own term    */
/* (an exact +0) included. One target per OpenMP iteration.                  */
/* ------------------------------------------------------------------------ */
void oracle_direct_fp32(const float *pos, const float *mass, int64_t n, float eps, const int64_t *targets,
                        int64_t n_targets, float *acc) {
    const float eps2 = eps * eps;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n_targets; t++) {
        const int64_t i = targets[t];
        const float xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
        float a[3] = {0.0f, 0.0f, 0.0f};
        for (int64_t j = 0; j < n; j++)
            add_term(mass[j], pos[3 * j] - xi, pos[3 * j + 1] - yi, pos[3 * j + 2] - zi, eps2, a);
        acc[3 * t + 0] = a[0];
        acc[3 * t + 1] = a[1];
        acc[3 * t + 2] = a[2];
    }
}

/* ------------------------------------------------------------------------ */
/* Accuracy reference ([PERF] "Accuracy"): the same softened force law       */
/* summed directly over all pairs in double precision, with Neumaier         */
/* compensation, for the listed targets (caller order). j = i is skipped.    */
/* ------------------------------------------------------------------------ */
typedef struct {
    double s, c;
} neumaier;

static void nm_add(neumaier *a, double x) {
    double t = a->s + x;
    if (fabs(a->s) >= fabs(x))
        a->c += (a->s - t) + x;
    else
        a->c += (x - t) + a->s;
    a->s = t;
}

void oracle_direct_fp64(const float *pos, const float *mass, int64_t n, double eps, const int64_t *targets,
                        int64_t n_targets, double *acc) {
    double eps2 = eps * eps;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n_targets; t++) {
        int64_t i = targets[t];
        double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
        neumaier ax = {0, 0}, ay = {0, 0}, az = {0, 0};
        for (int64_t j = 0; j < n; j++) {
            if (j == i) continue;
            double dx = (double)pos[3 * j] - xi, dy = (double)pos[3 * j + 1] - yi,
                   dz = (double)pos[3 * j + 2] - zi;
            double r2 = dx * dx + dy * dy + dz * dz + eps2;
            double f = (double)mass[j] / (r2 * sqrt(r2));
            nm_add(&ax, f * dx);
            nm_add(&ay, f * dy);
            nm_add(&az, f * dz);
        }
        acc[3 * t + 0] = ax.s + ax.c;
        acc[3 * t + 1] = ay.s + ay.c;
        acc[3 * t + 2] = az.s + az.c;
    }
}
