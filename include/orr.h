/*
 * orr.h - C ABI of liborr.so, the MI355X (gfx950) Barnes-Hut force evaluation.
 *
 * What it computes (the orrery pages):
 *   - "sycl_tree_solver.hpp" page, "The mitigation" and "What is not given
 *     up": a Barnes-Hut tree walk in which a 64-lane wave walks one shared
 *     node index; a lane that accepts a cell adds the cell's monopole term and
 *     then contributes nothing until the wave leaves that cell's subtree, so
 *     each target sums exactly the nodes its own walk visits, in the same
 *     order; enum TreeTraversal: the independent per-lane walk is kept as the
 *     measured baseline.
 *   - ADR-0029 "Mask the accepted cells rather than descending together",
 *     Decision: the wave advances to the smallest node index any lane still
 *     wants; Consequences: both traversals are the same function of the
 *     input, and interaction counts equal the CPU walk's.
 *   - performance page "docs/performance/sycl_tree.md", table "The machine and
 *     the device": softened monopole gravity (softening 0.05), opening angle
 *     0.5, leaf capacity 32; table "Where one evaluation goes": Morton sort,
 *     gather, build, node staging, walk, scatter. All of these steps run on
 *     the device here.
 *
 * Definitions used by every entry point (G = 1, float32 throughout):
 *   root cube: corner lo = component-wise minimum of the positions, side L =
 *     the largest per-axis extent (1 if that is 0); keys: 21 bits per axis,
 *     q = min(trunc((x - lo) * (2^21 / L)), 2^21 - 1), interleaved x-major
 *     into 63 bits; order: keys ascending, equal keys by ascending index;
 *   tree: a node of level l is a maximal run of sorted keys sharing their top
 *     3l bits; it splits iff it holds more than leaf_cap particles and l < 21;
 *     children are the non-empty octants in digit order; nodes are numbered in
 *     depth-first preorder (first child = index + 1) and escape = index +
 *     subtree size; node side s = L * 2^-l;
 *   moments: leaf M and S = sum m*x over its particles in sorted order,
 *     internal M and S = sum over children in octant order, com = S / M (the
 *     node's first particle if M = 0);
 *   walk of target i: at node c, accept iff s^2 < theta^2 * |com - x_i|^2;
 *     accept -> monopole term, pc += 1, go to escape; otherwise a leaf -> the
 *     term of each of its particles in sorted order, pp += its count minus the
 *     target itself, go to escape; otherwise -> c + 1;
 *   term: a += m * d * (|d|^2 + eps^2)^(-3/2), d = source - target, evaluated
 *     as r2 = ((dx*dx + dy*dy) + dz*dz) + eps^2, inv = 1/sqrt(r2),
 *     f = m * ((inv*inv)*inv), a += f*d, each step one correctly rounded
 *     float operation (no contraction), so results are reproducible bit for
 *     bit and identical between the two traversals.
 *
 * Conventions:
 *   - Array arguments are DEVICE pointers (HIP), contiguous, owned by the
 *     caller; positions are [n][3] float, masses [n] float, and every output
 *     is in the caller's particle order. Any output pointer may be NULL, in
 *     which case that output is not written.
 *   - The caller provides one device workspace of at least
 *     orr_workspace_bytes(n, leaf_cap) bytes, 256-byte aligned. The library
 *     allocates no device memory. The workspace holds the tree: it must stay
 *     alive and untouched while a tree handle that uses it is in use.
 *   - All device work is enqueued on the given HIP stream (NULL = the default
 *     stream) in stream order. No call synchronises the stream unless it says
 *     so.
 *   - Every entry point returns a status; nothing aborts and no C++ exception
 *     crosses the ABI. On error, orr_last_error() gives a thread-local
 *     message; outputs are then unspecified. Argument checks happen before any
 *     device work.
 *   - Fault injection (tests of the error paths): when the environment
 *     variable ORR_FAULT_INJECT names a site ("events", "cube", "sort",
 *     "build", "moments", "walk", "sync", "scratch", "direct", "alloc"), the
 *     entry points report a failure there (ORR_ERR_HIP, or
 *     ORR_ERR_HOST_MEMORY for "alloc") instead of calling HIP or allocating.
 *   - Node addressing (tests of the large-tree path): the coherent walk
 *     kernel addresses the node records by 32-bit byte offsets when the workspace's
 *     node bound (orr_workspace_bytes) fits in 4 GiB, about 82 million
 *     particles at leaf capacity 32, and by 64-bit indices above. Setting the
 *     environment variable ORR_WALK_NODE_OFFSETS to "64" makes every launch of
 *     it take the 64-bit path; results are the same bit for bit.
 *   - Checked build: liborr_checked.so exports this same ABI from the same
 *     sources compiled with ORR_CHECKED=1. Its kernels test every index they
 *     take from device data (node escapes, leaf ranges, the permutation, the
 *     sort's gather and run positions, the build's node slots and lists)
 *     against the array it addresses, skip an access that fails, and record
 *     the failure; the next call that synchronises (as for non-finite input,
 *     below) then returns ORR_ERR_HIP. It is about a quarter slower.
 *   - Inputs whose positions or masses are non-finite, whose masses are
 *     negative, or whose extent overflows float32 are detected on the device
 *     while the tree is built; the evaluation still runs to completion on a
 *     well-formed (but meaningless) tree, and the condition is reported as
 *     ORR_ERR_NONFINITE by the next call that synchronises (orr_tree_info_get,
 *     orr_tree_check, orr_workspace_check, or orr_eval_forces and
 *     orr_tree_walk with timings requested).
 */
#ifndef ORR_H
#define ORR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORR_ABI_VERSION 2
#define ORR_MAX_LEAF_CAP 256
#define ORR_MAX_N 2147483647LL

typedef enum {
    ORR_OK = 0,
    ORR_ERR_INVALID_ARG = 1, /* null pointer, bad enum, bad alignment */
    ORR_ERR_RANGE = 2,       /* n, leaf_cap, eps or theta out of range */
    ORR_ERR_NONFINITE = 3,   /* non-finite input found on the device */
    ORR_ERR_HIP = 4,         /* a HIP runtime call failed */
    ORR_ERR_WORKSPACE = 5,   /* workspace smaller than orr_workspace_bytes */
    ORR_ERR_HOST_MEMORY = 6  /* a host allocation (the tree handle) failed */
} orr_status;

/* Which walk the device runs (enum TreeTraversal of the solver page). */
typedef enum {
    ORR_TRAVERSAL_INDEPENDENT = 0, /* one lane per target, own node index */
    ORR_TRAVERSAL_COHERENT = 1     /* one node index per 64-lane wave, masked */
} orr_traversal;

typedef struct orr_tree orr_tree; /* host handle; device data lives in the workspace */

/* Where one evaluation spent its time, in milliseconds, measured with HIP
 * events on the stream (struct SyclTreeTimings of the solver page; phases of
 * the performance page's "Where one evaluation goes" table). */
typedef struct {
    float cube_keys_ms; /* root cube and Morton keys */
    float sort_ms;      /* radix sort of (key, index) */
    float gather_ms;    /* particles into sorted order: done inside the sort (its run fix-up), so 0 (in sort_ms) */
    float build_ms;     /* topology and escape indices (node staging included) */
    float moments_ms;   /* monopole moments */
    float walk_ms;      /* the traversal, scatter to caller order included */
    float scatter_ms;   /* outputs into caller order: done by the walk's stores, so 0 (in walk_ms) */
    float total_ms;
} orr_timings;

typedef struct {
    uint32_t n;
    uint32_t n_nodes;
    uint32_t n_leaves;
    uint32_t depth;          /* deepest node level */
    uint32_t max_leaf_count; /* may exceed leaf_cap only at level 21 */
    int32_t leaf_cap;
    float lo[3];
    float side;
    int32_t input_status;    /* ORR_OK or ORR_ERR_NONFINITE */
} orr_tree_info;

/* ABI version of the loaded library (ORR_ABI_VERSION it was built with). */
int orr_abi_version(void);

/* Static strings; never NULL. */
const char *orr_status_string(orr_status s);
const char *orr_traversal_name(orr_traversal t); /* "independent", "coherent", "invalid" */

/* Message of the last failure on the calling thread ("" if none). */
const char *orr_last_error(void);

/* Workspace bytes needed for n particles at this leaf capacity; 0 if the
 * arguments are out of range. Needs no GPU. The bound allows n leaves plus,
 * on each of the 21 split levels, n / (leaf_cap + 1) internal nodes. Node
 * indices are 32-bit, so that bound, n + 21 floor(n / (leaf_cap + 1)) + 1,
 * must not exceed 2^32 - 1: no limit below ORR_MAX_N at leaf capacities of
 * 20 and more, about 373 million particles at leaf capacity 1. Sizes beyond
 * it are out of range here and ORR_ERR_RANGE for every entry point that
 * takes n and leaf_cap. */
size_t orr_workspace_bytes(int64_t n, int32_t leaf_cap);

/* Enqueue the tree build: root cube, keys, sort, gather, topology, escape
 * indices and moments. pos [n][3], mass [n]. On success *out receives a host
 * handle (free with orr_tree_free) that refers to the workspace and stream.
 * Errors: ORR_ERR_INVALID_ARG (null pos/mass/workspace/out, workspace not
 * 256-byte aligned), ORR_ERR_RANGE (n < 1 or n > ORR_MAX_N, leaf_cap < 1 or
 * > ORR_MAX_LEAF_CAP, or a node bound beyond 32-bit indices: see
 * orr_workspace_bytes), ORR_ERR_WORKSPACE, ORR_ERR_HIP. */
orr_status orr_build_tree(const float *pos, const float *mass, int64_t n, int32_t leaf_cap,
                          void *workspace, size_t workspace_bytes, void *hip_stream, orr_tree **out);

/* Enqueue a walk over a built tree, on the tree's stream.
 * eps: finite and large enough that eps^-3, evaluated as the term evaluates
 * it (the cube of RN(1 / RN(sqrt(RN(eps * eps))))), is a finite float: the
 * target's own term is m * 0 * eps^-3 (d = 0) and is +0 only then (0 * inf
 * would make every acceleration NaN). In practice eps >= 1.43e-13. Results
 * are finite only where m * eps^-3 stays within float range for the masses m.
 * theta >= 0 and finite.
 * acc [n][3]; visits_own = nodes where the target's own walk acted (equal for
 * both traversals); visits_stepped = nodes its wave stepped through (the
 * union of the wave's walks for the coherent traversal, the own walk for the
 * independent one); n_pp = particle terms (self excluded), n_pc = accepted
 * cells. timings (HOST, may be NULL): if given, the walk is timed with HIP
 * events (walk_ms = total_ms; the other phases 0), the stream is
 * synchronised and the build's input status checked (ORR_ERR_NONFINITE
 * possible). Errors: ORR_ERR_INVALID_ARG (null tree, bad traversal),
 * ORR_ERR_RANGE (eps, theta), ORR_ERR_HIP. */
orr_status orr_tree_walk(const orr_tree *tree, float eps, float theta, orr_traversal traversal,
                         float *acc, uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                         uint32_t *n_pc, orr_timings *timings);

/* The walk with groups of group_width consecutive sorted targets (1, 2, 4,
 * ..., 64) sharing one node index: the sub-group coherence of the solver page
 * at any width (the performance page's "The sub-group width" compares 16 and
 * 32). A group steps through the union of its members' walks; node records
 * and leaf particles come through per-lane loads. group_width = 1 is the
 * independent walk. acc, visits_own, n_pp and n_pc are those of
 * orr_tree_walk (identical for every width); visits_stepped = size of the
 * union over the target's group. Errors: those of orr_tree_walk, and
 * ORR_ERR_RANGE for a group_width that is not a power of two in [1, 64]. */
orr_status orr_tree_walk_grouped(const orr_tree *tree, float eps, float theta, int32_t group_width,
                                 float *acc, uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                                 uint32_t *n_pc);

/* The coherent walk of orr_tree_walk with the wave's next node found as the
 * minimum of its lanes' next nodes (the advance the solver page describes
 * for its sub-groups, "The mitigation"): every lane keeps its own next node
 * and the wave takes a DPP minimum over them at every step, where
 * orr_tree_walk selects between c + 1 and the escape from the mask of
 * opening lanes. Both rules visit the same nodes in the same order, so every
 * output equals the coherent orr_tree_walk's bit for bit; this entry exists
 * to measure the reduction's cost. Arguments, outputs and errors as
 * orr_tree_walk with traversal = ORR_TRAVERSAL_COHERENT. */
orr_status orr_tree_walk_min_advance(const orr_tree *tree, float eps, float theta, float *acc,
                                     uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                                     uint32_t *n_pc);

/* The coherent walk of orr_tree_walk at coherence width 32, 64, 128 or 256
 * with the production walk's machinery (node records through scalar loads,
 * opened leaves staged in LDS and packed across the wave): the performance
 * page's "The sub-group width" question (16 against 32 lanes; would 64 pay)
 * and the work-group coherence of ADR-0029, "Alternatives considered".
 * width 32: each 64-lane wave holds two groups of 32 consecutive sorted
 * targets, each with its own node index; 64: orr_tree_walk itself; 128 and
 * 256: 2 or 4 waves of one work-group share one node index, agreed through
 * LDS at one barrier per step. acc, visits_own, n_pp and n_pc equal
 * orr_tree_walk's bit for bit at every width; visits_stepped = size of the
 * union of the walks of the target's group of `width` consecutive sorted
 * targets. Errors: those of orr_tree_walk, and ORR_ERR_RANGE for another
 * width (or a node array beyond 4 GiB). */
orr_status orr_tree_walk_width(const orr_tree *tree, float eps, float theta, int32_t width, float *acc,
                               uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc);

/* The alternative ADR-0029 rejects ("Alternatives considered"), the
 * published warp-coherent traversal, for comparison: groups of group_width
 * consecutive sorted targets (1, 2, 4, ..., 64) share one node; the group
 * opens a node when any member would, every member descending with it (at a
 * leaf, summing its particles), and otherwise every member adds the node's
 * term and the group skips the subtree. A target's sum then depends on its
 * group; group_width = 1 gives the walk of orr_tree_walk. Outputs as in
 * orr_tree_walk, with n_pp and n_pc of this walk and visits_own =
 * visits_stepped = nodes the group visited. Errors: as orr_tree_walk_grouped. */
orr_status orr_tree_walk_descend(const orr_tree *tree, float eps, float theta, int32_t group_width, float *acc,
                                 uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                                 uint32_t *n_pc);

/* The walk of orr_tree_walk over one contiguous range of sorted targets,
 * [first, first + count): the share of the targets one GPU walks when they
 * are split over several (given the tree, every target's walk is
 * independent of the others: ADR-0029, Consequences). The range holds whole
 * waves: first is a multiple of 64, and so is count unless first + count = n;
 * count = 0 (any first in [0, n]) enqueues nothing. Outputs are written for the range's targets
 * only, at their caller indices, bit for bit as orr_tree_walk writes them
 * (visits_stepped included, since every wave of the range is whole); all
 * other elements are left as they were. The coherent traversal orders the
 * range's waves by the rule of the whole walk's schedule, with one more
 * small kernel over the range; that schedule lives in the tree's workspace
 * until the next range walk of the tree, so range walks of one tree run one
 * at a time in stream order (the tree's stream). Errors: those of
 * orr_tree_walk, and ORR_ERR_RANGE for a range outside [0, n] or not made of
 * whole waves. */
orr_status orr_tree_walk_range(const orr_tree *tree, float eps, float theta, orr_traversal traversal,
                               int64_t first, int64_t count, float *acc, uint32_t *visits_own,
                               uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc);

/* Split the sorted targets into k contiguous ranges of whole waves with
 * nearly equal estimated walk cost, for orr_tree_walk_range: the cost of a
 * wave is the estimate the coherent walk's schedule orders waves by (summed
 * leaf depth of its 64 targets plus 32 per level between its deepest leaf and
 * the smallest cell holding all of them). bounds (HOST memory, k + 1 int64)
 * receives 0 = bounds[0] <= bounds[1] <= ... <= bounds[k] = n; range j is
 * [bounds[j], bounds[j + 1]), bound j the first wave boundary at which the
 * cost before it reaches j / k of the total. Synchronises the tree's stream.
 * Errors: ORR_ERR_INVALID_ARG (null pointer), ORR_ERR_RANGE (k < 1 or
 * k > 65536), ORR_ERR_HIP. */
orr_status orr_tree_shard_bounds(const orr_tree *tree, int32_t k, int64_t *bounds);

/* Build and walk in one call. If timings is not NULL, every phase is timed
 * with HIP events, the stream is synchronised and the input status checked
 * (ORR_ERR_NONFINITE possible). Errors: those of orr_build_tree and
 * orr_tree_walk. */
orr_status orr_eval_forces(const float *pos, const float *mass, int64_t n, float eps, float theta,
                           int32_t leaf_cap, orr_traversal traversal, float *acc, uint32_t *visits_own,
                           uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc, void *workspace,
                           size_t workspace_bytes, void *hip_stream, orr_timings *timings);

/* Bytes of the fixed device array that orr_eval_forces_noalloc uses as its
 * workspace: 144 MiB per GPU, enough for n = 1,048,576 at leaf_cap 32 (any
 * (n, leaf_cap) with orr_workspace_bytes(n, leaf_cap) <= this). */
#define ORR_NOALLOC_SCRATCH_BYTES (144ull << 20)

/* orr_eval_forces for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same evaluation, outputs and errors, with the workspace
 * taken from a fixed array of ORR_NOALLOC_SCRATCH_BYTES in the library's own
 * device memory instead of a caller's buffer, and no timings. It calls no
 * device allocation or free: the array is part of the library's code object
 * on each GPU, from its loading until the process ends, and is looked up once
 * per device on the first call (with that device current; the stream must
 * belong to the current device). The caller still passes inputs and outputs
 * (device pointers). Every call on one GPU uses that GPU's one array, so calls
 * that overlap on one GPU (on different streams, or from several threads
 * without ordering) race and give undefined results; calls in one stream's
 * order are safe. Errors: those of orr_eval_forces, and ORR_ERR_WORKSPACE when
 * orr_workspace_bytes(n, leaf_cap) > ORR_NOALLOC_SCRATCH_BYTES. */
orr_status orr_eval_forces_noalloc(const float *pos, const float *mass, int64_t n, float eps, float theta,
                                   int32_t leaf_cap, orr_traversal traversal, float *acc, uint32_t *visits_own,
                                   uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc, void *hip_stream);

/* Status of the most recent evaluation or build in this workspace, for
 * callers of orr_eval_forces without timings (which returns before the
 * device has looked at the input): synchronises hip_stream (the stream that
 * evaluation used) and reads the workspace's parameter block. ORR_OK;
 * ORR_ERR_NONFINITE if that input was non-finite or had a negative mass;
 * ORR_ERR_HIP if a bounded wait of its radix sort gave up (never expected;
 * its outputs are then invalid), or, in the checked build, if a device
 * index check failed. Every build resets the status, so a caller
 * that evaluates several times checks after each evaluation it relies on.
 * Errors: ORR_ERR_INVALID_ARG (null or unaligned workspace),
 * ORR_ERR_WORKSPACE (smaller than its parameter block), ORR_ERR_HIP. */
orr_status orr_workspace_check(const void *workspace, size_t workspace_bytes, void *hip_stream);

/* Synchronise the tree's stream and report its sizes and input status.
 * Returns ORR_ERR_NONFINITE (with *out filled) if the input was non-finite. */
orr_status orr_tree_info_get(const orr_tree *tree, orr_tree_info *out);

/* Synchronise the stream of a previous build in this workspace and report
 * its input status (ORR_OK or ORR_ERR_NONFINITE). */
orr_status orr_tree_check(const orr_tree *tree);

/* Enqueue device-to-device copies of the tree for inspection. Sizes: n for
 * keys_sorted (uint64) and perm (uint32, sorted position -> caller index);
 * n_nodes (from orr_tree_info_get) for level (uint8), begin, count, escape
 * (uint32), geom ([n_nodes][4] float: com x, y, z, mass) and s2 (float, the
 * squared node side). Any pointer may be NULL. */
orr_status orr_tree_export(const orr_tree *tree, uint64_t *keys_sorted, uint32_t *perm, uint8_t *level,
                           uint32_t *begin, uint32_t *count, uint32_t *escape, float *geom, float *s2);

/* Enqueue device-to-device copies of the coherent walk's schedule, which the
 * tree build computes and which decides only when each target wave runs, never
 * what it computes (the orrery solver page, "The mitigation": waves of 64
 * consecutive sorted targets). wave_cost [n_waves] (n_waves = ceil(n / 64),
 * uint32): a wave's estimated run time, its targets' summed leaf level plus 32
 * times the levels between its deepest leaf and the smallest cell holding all
 * its targets. order [64 ceil(n_waves / 64) + 8] (uint32): eight lists of
 * waves, one per XCD, list x at order[x L ..], L = 8 ceil(n_waves / 64), its
 * length at order[8 L + x]; entries past a list's length are unspecified.
 * Either pointer may be NULL. Errors: ORR_ERR_INVALID_ARG (NULL tree),
 * ORR_ERR_HIP. */
orr_status orr_tree_export_schedule(const orr_tree *tree, uint32_t *wave_cost, uint32_t *order);

/* All-pairs float32 direct sum, the reference the tree is measured against
 * (the direct solver of the orrery performance page, "Against the two solvers
 * it has to beat"): for every particle i, acc[i] = sum over j = 0..n-1 in
 * index order of the walk's softened term m_j d (|d|^2 + eps^2)^(-3/2),
 * d = x_j - x_i, each step one correctly rounded float32 operation (the
 * particle's own term is +0). O(n^2) work. pos [n][3], mass [n], acc [n][3]:
 * device pointers, caller-owned; enqueued on hip_stream; no workspace.
 * Errors: ORR_ERR_INVALID_ARG (null pointer), ORR_ERR_RANGE (n < 1 or
 * n > ORR_MAX_N, eps outside the range of orr_tree_walk), ORR_ERR_HIP. */
orr_status orr_direct_forces(const float *pos, const float *mass, int64_t n, float eps, float *acc,
                             void *hip_stream);

/* The all-pairs float32 direct sum of orr_direct_forces for selected targets
 * only, the accuracy reference at sizes where the whole O(n^2) sum costs too
 * much (the performance page's "Accuracy" measures the tree against a direct
 * sum): acc[t] ([n_targets][3]) = the sum over j = 0..n-1 in index order for
 * the particle with caller index targets[t], bit for bit what
 * orr_direct_forces gives that particle. targets: DEVICE int64 [n_targets],
 * caller indices; an index outside [0, n) yields NaN in its row (the
 * device cannot report it without a synchronisation) and reads nothing.
 * O(n n_targets) work. Errors: ORR_ERR_INVALID_ARG (null pointer),
 * ORR_ERR_RANGE (n, n_targets < 0 or > ORR_MAX_N, eps as orr_tree_walk),
 * ORR_ERR_HIP. */
orr_status orr_direct_forces_targets(const float *pos, const float *mass, int64_t n, float eps, const int64_t *targets,
                                     int64_t n_targets, float *acc, void *hip_stream);

/* The accuracy reference of the performance page ("Accuracy": the same
 * softened force law summed with compensation in double precision), for
 * selected targets: acc[t] ([n_targets][3], DEVICE double) = sum over every
 * other particle j != i, in index order, of m_j d (r2 sqrt(r2))^-1 with
 * d = x_j - x_i and r2 = dx*dx + dy*dy + dz*dz + eps^2 in IEEE double
 * operations, each component summed with Neumaier's compensation, for the
 * caller index i = targets[t] (DEVICE int64; outside [0, n): NaN, nothing
 * read). The self term is left out, so eps = 0 is allowed. O(n n_targets)
 * work. Errors: ORR_ERR_INVALID_ARG (null pointer), ORR_ERR_RANGE (n,
 * n_targets < 0 or > ORR_MAX_N, eps negative or not finite), ORR_ERR_HIP. */
orr_status orr_direct_forces_fp64_targets(const float *pos, const float *mass, int64_t n, double eps,
                                          const int64_t *targets, int64_t n_targets, double *acc, void *hip_stream);

/* Self-check of the walk's inverse square root. For eps >= 2^-48 the walk
 * evaluates RN(1/RN(sqrt(r2))) with a shorter instruction sequence valid for
 * r2 >= 2^-96 (every r2 >= eps^2 there); this enqueues a comparison of that
 * sequence with the IEEE square root and division for every float whose bit
 * pattern lies in [first_bits, last_bits]. *mismatches (device, uint64)
 * receives the count and examples (device, 8 x uint32) up to 8 failing bit
 * patterns. Errors: ORR_ERR_INVALID_ARG (null pointer, first > last),
 * ORR_ERR_HIP. */
orr_status orr_selftest_inv_sqrt(uint32_t first_bits, uint32_t last_bits, uint64_t *mismatches,
                                 uint32_t *examples, void *hip_stream);

/* Release the host handle. The workspace stays the caller's. NULL is a no-op. */
void orr_tree_free(orr_tree *tree);

#ifdef __cplusplus
}
#endif

#endif /* ORR_H */
