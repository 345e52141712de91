// C ABI of liborr (declared in include/orr.h): argument checks, workspace
// layout, and the stream-ordered sequence of kernels of one evaluation.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "orr.h"
#include "orr_internal.h"
#include "schedule.h"

namespace orr {

namespace {

thread_local std::string g_last_error;

orr_status fail(orr_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
orr_status fail(orr_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

orr_status hip_fail(hipError_t e, const char *where) {
    return fail(ORR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Fault injection, for tests of the error paths on any machine: when the
// environment variable ORR_FAULT_INJECT names a site, that site reports a
// failure instead of calling HIP (or allocating). Sites: "events" (timing
// events), "cube", "sort", "build", "moments", "walk" (every walk launch),
// "sync" (reading the device parameters back), "scratch" (the
// allocation-free entry's set-up), "direct", "alloc" (the host tree handle).
bool injected(const char *site) {
    const char *v = std::getenv("ORR_FAULT_INJECT");
    return v && std::strcmp(v, site) == 0;
}

hipError_t maybe_fault(const char *site) { return injected(site) ? hipErrorLaunchFailure : hipSuccess; }

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// The int a C caller passed for an enum argument, read from the argument's
// bytes: any int may arrive there, and loading a value outside the enum's
// range through the enum type itself would be undefined in C++.
template <class E>
int enum_bits(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

}  // namespace

size_t carve_workspace(void *base, int64_t n, int32_t leaf_cap, Workspace *ws) {
    const int64_t nb = max_nodes_for(n, leaf_cap);
    const int64_t n_tiles = ceil_div(n, sort_tile_keys(n));
    const int64_t n_scan_tiles = ceil_div(n + 1, 256);
    char *p = static_cast<char *>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *r = p ? p + off : nullptr;
        off = align_up(off + bytes);
        return r;
    };
    Workspace w{};
    w.prm = reinterpret_cast<DevParams *>(take(sizeof(DevParams)));
    w.cube_part = reinterpret_cast<float *>(take(sizeof(float) * 8 * kCubeBlocks));
    for (int k = 0; k < 2; k++) w.keys[k] = reinterpret_cast<uint64_t *>(take(sizeof(uint64_t) * n));
    for (int k = 0; k < 2; k++) w.vals[k] = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * n));
    w.hist_part = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * kSortHistBlocks * kRadixPasses * kRadixBins));
    w.digit_offs = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * kRadixPasses * kRadixBins));
    w.n_lb_words = (int64_t)kFullPasses * n_tiles * kRadixBins;
    w.lb_words = reinterpret_cast<uint64_t *>(take(sizeof(uint64_t) * w.n_lb_words));
    w.xs = reinterpret_cast<float4 *>(take(sizeof(float4) * n));
    w.info = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * n));
    w.base = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * (n + 1)));
    w.tile_sum = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * (n_scan_tiles + 1)));
    w.nodes = reinterpret_cast<NodeRec *>(take(sizeof(NodeRec) * nb));
    w.msum = reinterpret_cast<float4 *>(take(sizeof(float4) * nb));
    w.level = reinterpret_cast<uint8_t *>(take(sizeof(uint8_t) * nb));
    w.cut_list = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * nb));
    w.max_top = max_top_for(n);
    w.top_list = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * w.max_top));
    w.kids = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * 9 * w.max_top));
    w.n_waves = ceil_div(n, 64);
    w.wave_cost = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * w.n_waves));
    w.wave_order = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * schedule_slots(w.n_waves)));
    w.range_order = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * schedule_slots(w.n_waves)));
    w.n = n;
    w.leaf_cap = leaf_cap;
    w.max_nodes = nb;
    w.n_tiles = n_tiles;
    if (ws) *ws = w;
    return off;
}

}  // namespace orr

using namespace orr;

struct orr_tree {
    Workspace ws;
    hipStream_t stream;
};

namespace {

// Node indices, escapes and node counts are 32-bit on the device, so the
// workspace's node bound must stay below 2^32 (it does for every n <=
// ORR_MAX_N at leaf capacities of 20 and more; at capacity 1 up to about 373
// million particles).
bool node_bound_fits(int64_t n, int32_t leaf_cap) { return max_nodes_for(n, leaf_cap) <= (int64_t)0xffffffffll; }

bool valid_sizes(int64_t n, int32_t leaf_cap) {
    return n >= 1 && n <= ORR_MAX_N && leaf_cap >= 1 && leaf_cap <= ORR_MAX_LEAF_CAP && node_bound_fits(n, leaf_cap);
}

orr_status check_sizes(int64_t n, int32_t leaf_cap) {
    if (n < 1 || n > ORR_MAX_N) return fail(ORR_ERR_RANGE, "n = %lld is outside [1, %lld]", (long long)n, ORR_MAX_N);
    if (leaf_cap < 1 || leaf_cap > ORR_MAX_LEAF_CAP)
        return fail(ORR_ERR_RANGE, "leaf_cap = %d is outside [1, %d]", leaf_cap, ORR_MAX_LEAF_CAP);
    if (!node_bound_fits(n, leaf_cap))
        return fail(ORR_ERR_RANGE, "n = %lld at leaf_cap = %d allows more than 2^32 - 1 nodes (32-bit node indices)",
                    (long long)n, leaf_cap);
    return ORR_OK;
}

// The target's own term is m * 0 * eps^-3 (d = 0). It is +0, as the force law
// wants, only while eps^-3 evaluated as the term evaluates it, the cube of
// RN(1 / RN(sqrt(RN(eps * eps)))), is finite; for smaller eps it is 0 * inf
// = NaN on every target. The bound lies near eps = 1.43e-13, where eps^2 is
// far above 2^-96, the lower end of the walk's inverse square root domain.
bool eps_in_range(float eps) {
    if (!(std::isfinite(eps) && eps > 0.0f)) return false;
    const float e2 = eps * eps;
    if (!(e2 >= 0x1p-96f)) return false;
    const float inv = 1.0f / std::sqrt(e2);
    return std::isfinite((inv * inv) * inv);
}

orr_status check_eps(float eps) {
    if (!eps_in_range(eps))
        return fail(ORR_ERR_RANGE, "eps must be finite with a finite float32 eps^-3, about eps >= 1.43e-13 (got %g)",
                    eps);
    return ORR_OK;
}

orr_status check_walk_args(float eps, float theta, int traversal) {
    if (check_eps(eps) != ORR_OK) return ORR_ERR_RANGE;
    if (!(std::isfinite(theta) && theta >= 0.0f))
        return fail(ORR_ERR_RANGE, "theta must be finite and >= 0 (got %g)", theta);
    if (traversal != ORR_TRAVERSAL_INDEPENDENT && traversal != ORR_TRAVERSAL_COHERENT)
        return fail(ORR_ERR_INVALID_ARG, "traversal %d is not a orr_traversal", traversal);
    return ORR_OK;
}

orr_status check_build_args(const float *pos, const float *mass, int64_t n, int32_t leaf_cap, void *workspace,
                            size_t workspace_bytes) {
    orr_status st = check_sizes(n, leaf_cap);
    if (st != ORR_OK) return st;
    if (!pos || !mass) return fail(ORR_ERR_INVALID_ARG, "pos and mass must not be NULL");
    if (!workspace) return fail(ORR_ERR_INVALID_ARG, "workspace must not be NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(ORR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t need = carve_workspace(nullptr, n, leaf_cap, nullptr);
    if (workspace_bytes < need)
        return fail(ORR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    return ORR_OK;
}

// Records an event on the stream if timing is on.
struct PhaseTimer {
    bool on = false;
    hipStream_t s = nullptr;
    hipEvent_t ev[8] = {};
    int k = 0;
    hipError_t init(bool enable, hipStream_t stream) {
        on = enable;
        s = stream;
        if (!on) return hipSuccess;
        if (injected("events")) return hipErrorOutOfMemory;
        for (auto &e : ev) {
            hipError_t r = hipEventCreate(&e);
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    }
    hipError_t mark() { return on ? hipEventRecord(ev[k++], s) : hipSuccess; }
    float ms(int a, int b) {
        float t = 0.0f;
        (void)hipEventElapsedTime(&t, ev[a], ev[b]);
        return t;
    }
    ~PhaseTimer() {
        for (auto &e : ev)
            if (e) (void)hipEventDestroy(e);
    }
};

// A roctx range around the host-side enqueue of one phase (rocprofv3
// --marker-trace shows it beside the phase's kernels); popped on every return.
struct Range {
    explicit Range(const char *name) { roctxRangePushA(name); }
    ~Range() { roctxRangePop(); }
    Range(const Range &) = delete;
    Range &operator=(const Range &) = delete;
};

// Phase marks: 0 start, 1 after cube and keys, 2 after sort and gather, 3
// after topology, 4 after moments, 5 after the walk.
orr_status build_into(const float *pos, const float *mass, const Workspace &ws, hipStream_t s, PhaseTimer &tm) {
    hipError_t e;
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    {
        Range r("orr: cube, keys, sort and gather");
        if ((e = maybe_fault("cube")) != hipSuccess || (e = launch_cube(pos, mass, ws, s)) != hipSuccess)
            return hip_fail(e, "root cube");
        if ((e = maybe_fault("sort")) != hipSuccess ||
            (e = launch_keys_and_sort(pos, mass, ws, s, tm.on ? tm.ev[tm.k++] : nullptr)) != hipSuccess)
            return hip_fail(e, "keys / radix sort");
    }
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    {
        Range r("orr: tree topology");
        if ((e = maybe_fault("build")) != hipSuccess || (e = launch_build(ws, s)) != hipSuccess)
            return hip_fail(e, "tree build");
    }
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    {
        Range r("orr: moments and walk schedule");
        if ((e = maybe_fault("moments")) != hipSuccess || (e = launch_moments(ws, s)) != hipSuccess)
            return hip_fail(e, "moments");
    }
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return ORR_OK;
}

orr_status read_params(const orr_tree *t, DevParams *out) {
    if (injected("sync")) return hip_fail(hipErrorIllegalAddress, "hipMemcpyAsync (injected)");
    hipError_t e = hipMemcpyAsync(out, t->ws.prm, sizeof(DevParams), hipMemcpyDeviceToHost, t->stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    if ((e = hipStreamSynchronize(t->stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (out->bad_input & 2u) return fail(ORR_ERR_HIP, "a device look-back wait gave up; results are invalid");
    if (out->bad_input & kBadIndex)
        return fail(ORR_ERR_HIP, "a device index check failed (index out of its array's range); results are invalid");
    return ORR_OK;
}

}  // namespace

#define ORR_GUARD_BEGIN try {
#define ORR_GUARD_END                                                       \
    }                                                                       \
    catch (const std::bad_alloc &) {                                        \
        return fail(ORR_ERR_HOST_MEMORY, "host allocation failed");         \
    }                                                                       \
    catch (...) {                                                           \
        return fail(ORR_ERR_INVALID_ARG, "unexpected C++ exception");      \
    }

extern "C" {

int orr_abi_version(void) { return ORR_ABI_VERSION; }

const char *orr_status_string(orr_status s) {
    switch (enum_bits(s)) {
        case ORR_OK: return "ok";
        case ORR_ERR_INVALID_ARG: return "invalid argument";
        case ORR_ERR_RANGE: return "argument out of range";
        case ORR_ERR_NONFINITE: return "non-finite or negative input";
        case ORR_ERR_HIP: return "HIP runtime error";
        case ORR_ERR_WORKSPACE: return "workspace too small";
        case ORR_ERR_HOST_MEMORY: return "host allocation failed";
    }
    return "unknown status";
}

const char *orr_traversal_name(orr_traversal t) {
    switch (enum_bits(t)) {
        case ORR_TRAVERSAL_INDEPENDENT: return "independent";
        case ORR_TRAVERSAL_COHERENT: return "coherent";
    }
    return "invalid";
}

const char *orr_last_error(void) { return g_last_error.c_str(); }

size_t orr_workspace_bytes(int64_t n, int32_t leaf_cap) {
    if (!valid_sizes(n, leaf_cap)) return 0;
    return carve_workspace(nullptr, n, leaf_cap, nullptr);
}

orr_status orr_build_tree(const float *pos, const float *mass, int64_t n, int32_t leaf_cap, void *workspace,
                          size_t workspace_bytes, void *hip_stream, orr_tree **out) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!out) return fail(ORR_ERR_INVALID_ARG, "out must not be NULL");
    *out = nullptr;
    orr_status st = check_build_args(pos, mass, n, leaf_cap, workspace, workspace_bytes);
    if (st != ORR_OK) return st;
    if (injected("alloc")) throw std::bad_alloc();
    orr_tree *t = new orr_tree;
    carve_workspace(workspace, n, leaf_cap, &t->ws);
    t->stream = static_cast<hipStream_t>(hip_stream);
    PhaseTimer tm;
    st = build_into(pos, mass, t->ws, t->stream, tm);
    if (st != ORR_OK) {
        delete t;
        return st;
    }
    *out = t;
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_walk(const orr_tree *tree, float eps, float theta, orr_traversal traversal, float *acc,
                         uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                         orr_timings *timings) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    orr_status st = check_walk_args(eps, theta, enum_bits(traversal));
    if (st != ORR_OK) return st;
    PhaseTimer tm;
    hipError_t e = tm.init(timings != nullptr, tree->stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    {
        Range r("orr: walk");
        e = maybe_fault("walk");
        if (e == hipSuccess)
            e = launch_walk(tree->ws, enum_bits(traversal) == ORR_TRAVERSAL_COHERENT ? kWalkCoherent : kWalkIndependent,
                            eps * eps, theta * theta, acc, visits_own, visits_stepped, n_pp, n_pc, tree->stream);
    }
    if (e != hipSuccess) return hip_fail(e, "walk");
    if (!timings) return ORR_OK;
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    DevParams prm;
    if ((st = read_params(tree, &prm)) != ORR_OK) return st;
    *timings = orr_timings{};
    timings->walk_ms = tm.ms(0, 1);
    timings->total_ms = timings->walk_ms;
    if (prm.bad_input) return fail(ORR_ERR_NONFINITE, "non-finite position or mass, or negative mass, in the input");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_walk_min_advance(const orr_tree *tree, float eps, float theta, float *acc, uint32_t *visits_own,
                                     uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    orr_status st = check_walk_args(eps, theta, ORR_TRAVERSAL_COHERENT);
    if (st != ORR_OK) return st;
    hipError_t e = maybe_fault("walk");
    if (e == hipSuccess)
        e = launch_walk(tree->ws, kWalkCoherentMin, eps * eps, theta * theta, acc, visits_own, visits_stepped,
                        n_pp, n_pc, tree->stream);
    if (e != hipSuccess) return hip_fail(e, "min-advance walk");
    return ORR_OK;
    ORR_GUARD_END
}

static orr_status walk_grouped_entry(const orr_tree *tree, float eps, float theta, int32_t group_width,
                                     bool descend, float *acc, uint32_t *visits_own,
                                     uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    orr_status st = check_walk_args(eps, theta, ORR_TRAVERSAL_COHERENT);
    if (st != ORR_OK) return st;
    if (group_width < 1 || group_width > 64 || (group_width & (group_width - 1)) != 0)
        return fail(ORR_ERR_RANGE, "group_width %d is not a power of two in [1, 64]", group_width);
    hipError_t e = maybe_fault("walk");
    if (e == hipSuccess)
        e = launch_walk_grouped(tree->ws, group_width, descend, eps * eps, theta * theta, acc, visits_own,
                                visits_stepped, n_pp, n_pc, tree->stream);
    if (e != hipSuccess) return hip_fail(e, descend ? "descend-together walk" : "grouped walk");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_walk_grouped(const orr_tree *tree, float eps, float theta, int32_t group_width,
                                 float *acc, uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                                 uint32_t *n_pc) {
    return walk_grouped_entry(tree, eps, theta, group_width, false, acc, visits_own, visits_stepped, n_pp, n_pc);
}

orr_status orr_tree_walk_descend(const orr_tree *tree, float eps, float theta, int32_t group_width, float *acc,
                                 uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                                 uint32_t *n_pc) {
    return walk_grouped_entry(tree, eps, theta, group_width, true, acc, visits_own, visits_stepped, n_pp, n_pc);
}

orr_status orr_tree_walk_width(const orr_tree *tree, float eps, float theta, int32_t width, float *acc,
                               uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    orr_status st = check_walk_args(eps, theta, ORR_TRAVERSAL_COHERENT);
    if (st != ORR_OK) return st;
    if (width != 32 && width != 64 && width != 128 && width != 256)
        return fail(ORR_ERR_RANGE, "width %d is not 32, 64, 128 or 256", width);
    if ((uint64_t)tree->ws.max_nodes * sizeof(NodeRec) > 0xffffffffull)
        return fail(ORR_ERR_RANGE, "n = %lld is too large for the width walks (node array beyond 4 GiB)",
                    (long long)tree->ws.n);
    hipError_t e = maybe_fault("walk");
    if (e == hipSuccess)
        e = launch_walk_width(tree->ws, width, eps * eps, theta * theta, acc, visits_own, visits_stepped,
                              n_pp, n_pc, tree->stream);
    if (e != hipSuccess) return hip_fail(e, "width walk");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_walk_range(const orr_tree *tree, float eps, float theta, orr_traversal traversal,
                               int64_t first, int64_t count, float *acc, uint32_t *visits_own,
                               uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    orr_status st = check_walk_args(eps, theta, enum_bits(traversal));
    if (st != ORR_OK) return st;
    const Workspace &ws = tree->ws;
    if (first < 0 || count < 0 || first > ws.n || count > ws.n - first)
        return fail(ORR_ERR_RANGE, "targets [%lld, %lld + %lld) are not inside [0, %lld)", (long long)first,
                    (long long)first, (long long)count, (long long)ws.n);
    if (count == 0) return ORR_OK;  // an empty range (bounds of orr_tree_shard_bounds may repeat n)
    if (first % 64 != 0 || (count % 64 != 0 && first + count != ws.n))
        return fail(ORR_ERR_RANGE, "targets [%lld, %lld + %lld) are not whole waves of 64", (long long)first,
                    (long long)first, (long long)count);
    hipError_t e;
    const bool coherent = enum_bits(traversal) == ORR_TRAVERSAL_COHERENT;
    if (coherent && (e = launch_range_schedule(ws, first / 64, ceil_div(count, 64), tree->stream)) != hipSuccess)
        return hip_fail(e, "range schedule");
    e = maybe_fault("walk");
    if (e == hipSuccess)
        e = launch_walk_range(ws, coherent ? kWalkCoherent : kWalkIndependent, WalkRange{first, count, ws.range_order},
                              eps * eps, theta * theta, acc, visits_own, visits_stepped, n_pp, n_pc, tree->stream);
    if (e != hipSuccess) return hip_fail(e, "range walk");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_shard_bounds(const orr_tree *tree, int32_t k, int64_t *bounds) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree || !bounds) return fail(ORR_ERR_INVALID_ARG, "tree and bounds must not be NULL");
    if (k < 1 || k > 65536) return fail(ORR_ERR_RANGE, "k = %d is outside [1, 65536]", k);
    const Workspace &ws = tree->ws;
    std::vector<uint32_t> cost((size_t)ws.n_waves);
    hipError_t e = hipMemcpyAsync(cost.data(), ws.wave_cost, cost.size() * sizeof(uint32_t),
                                  hipMemcpyDeviceToHost, tree->stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    if ((e = hipStreamSynchronize(tree->stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint64_t total = 0;
    for (uint32_t c : cost) total += c;
    // bound j: the first wave w with (cost of waves < w) * k >= j * total
    bounds[0] = 0;
    uint64_t before = 0;
    size_t w = 0;
    for (int32_t j = 1; j < k; j++) {
        while (w < cost.size() && before * (uint64_t)k < (uint64_t)j * total) before += cost[w++];
        bounds[j] = std::min<int64_t>((int64_t)w * 64, ws.n);
    }
    bounds[k] = ws.n;
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_eval_forces(const float *pos, const float *mass, int64_t n, float eps, float theta,
                           int32_t leaf_cap, orr_traversal traversal, float *acc, uint32_t *visits_own,
                           uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc, void *workspace,
                           size_t workspace_bytes, void *hip_stream, orr_timings *timings) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    orr_status st = check_build_args(pos, mass, n, leaf_cap, workspace, workspace_bytes);
    if (st != ORR_OK) return st;
    if ((st = check_walk_args(eps, theta, enum_bits(traversal))) != ORR_OK) return st;
    orr_tree t;
    carve_workspace(workspace, n, leaf_cap, &t.ws);
    t.stream = static_cast<hipStream_t>(hip_stream);
    PhaseTimer tm;
    hipError_t e = tm.init(timings != nullptr, t.stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((st = build_into(pos, mass, t.ws, t.stream, tm)) != ORR_OK) return st;
    {
        Range r("orr: walk");
        e = maybe_fault("walk");
        if (e == hipSuccess)
            e = launch_walk(t.ws, enum_bits(traversal) == ORR_TRAVERSAL_COHERENT ? kWalkCoherent : kWalkIndependent,
                            eps * eps, theta * theta, acc, visits_own, visits_stepped, n_pp, n_pc, t.stream);
    }
    if (e != hipSuccess) return hip_fail(e, "walk");
    if (!timings) return ORR_OK;
    if ((e = tm.mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    DevParams prm;
    if ((st = read_params(&t, &prm)) != ORR_OK) return st;
    timings->cube_keys_ms = tm.ms(0, 1);
    timings->sort_ms = tm.ms(1, 2);
    timings->gather_ms = 0.0f;  // done by the sort's run fix-up, inside sort_ms
    timings->build_ms = tm.ms(2, 3);
    timings->moments_ms = tm.ms(3, 4);
    timings->walk_ms = tm.ms(4, 5);
    timings->scatter_ms = 0.0f;  // the walk stores its outputs in caller order
    timings->total_ms = tm.ms(0, 5);
    if (prm.bad_input) return fail(ORR_ERR_NONFINITE, "non-finite position or mass, or negative mass, in the input");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_workspace_check(const void *workspace, size_t workspace_bytes, void *hip_stream) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!workspace) return fail(ORR_ERR_INVALID_ARG, "workspace must not be NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(ORR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < sizeof(DevParams))
        return fail(ORR_ERR_WORKSPACE, "workspace has %zu bytes, fewer than one build's parameters", workspace_bytes);
    orr_tree t;
    t.ws = Workspace{};
    t.ws.prm = static_cast<DevParams *>(const_cast<void *>(workspace));  // the workspace starts with them
    t.stream = static_cast<hipStream_t>(hip_stream);
    DevParams prm;
    orr_status st = read_params(&t, &prm);
    if (st != ORR_OK) return st;
    if (prm.bad_input) return fail(ORR_ERR_NONFINITE, "non-finite position or mass, or negative mass, in the input");
    return ORR_OK;
    ORR_GUARD_END
}

}  // extern "C"

// Workspace of orr_eval_forces_noalloc: one fixed array in device memory per
// GPU, loaded with the library's code object and held until the process
// ends. In host code `scratch` names a host-side stand-in, never the device
// memory: every host use goes through the address hipGetSymbolAddress returns
// for the current device (kept per device in g_scratch_ptr).
static __device__ __align__(256) unsigned char scratch[ORR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
orr_status scratch_for_current_device(void **out) {
    int dev = -1;
    hipError_t e = injected("scratch") ? hipErrorNoDevice : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ORR_ERR_HIP, "device %d is beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
            return fail(ORR_ERR_HIP, "scratch array of device %d is not 256-byte aligned", dev);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ORR_OK;
}

}  // namespace

extern "C" {

orr_status orr_eval_forces_noalloc(const float *pos, const float *mass, int64_t n, float eps, float theta,
                                   int32_t leaf_cap, orr_traversal traversal, float *acc, uint32_t *visits_own,
                                   uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc, void *hip_stream) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    orr_status st = check_sizes(n, leaf_cap);
    if (st != ORR_OK) return st;
    const size_t need = carve_workspace(nullptr, n, leaf_cap, nullptr);
    if (need > (size_t)ORR_NOALLOC_SCRATCH_BYTES)
        return fail(ORR_ERR_WORKSPACE,
                    "n = %lld at leaf_cap %d needs %zu bytes of workspace; the allocation-free entry holds %zu",
                    (long long)n, leaf_cap, need, (size_t)ORR_NOALLOC_SCRATCH_BYTES);
    if (!pos || !mass) return fail(ORR_ERR_INVALID_ARG, "pos and mass must not be NULL");
    if ((st = check_walk_args(eps, theta, enum_bits(traversal))) != ORR_OK) return st;
    void *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != ORR_OK) return st;
    // the evaluation without timings enqueues kernels only (no allocation,
    // fill, copy or host wait), and those kernels initialise every part of
    // the workspace they read before reading it
    return orr_eval_forces(pos, mass, n, eps, theta, leaf_cap, traversal, acc, visits_own, visits_stepped, n_pp,
                           n_pc, ws, (size_t)ORR_NOALLOC_SCRATCH_BYTES, hip_stream, nullptr);
    ORR_GUARD_END
}

orr_status orr_tree_info_get(const orr_tree *tree, orr_tree_info *out) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree || !out) return fail(ORR_ERR_INVALID_ARG, "tree and out must not be NULL");
    hipError_t e = launch_tree_info(tree->ws, tree->stream);
    if (e != hipSuccess) return hip_fail(e, "tree info");
    DevParams prm;
    orr_status st = read_params(tree, &prm);
    if (st != ORR_OK) return st;
    out->n = (uint32_t)tree->ws.n;
    out->n_nodes = prm.n_nodes;
    out->n_leaves = prm.n_leaves;
    out->depth = prm.depth;
    out->max_leaf_count = prm.max_leaf_count;
    out->leaf_cap = tree->ws.leaf_cap;
    for (int a = 0; a < 3; a++) out->lo[a] = prm.lo[a];
    out->side = prm.side;
    out->input_status = prm.bad_input ? ORR_ERR_NONFINITE : ORR_OK;
    if (prm.bad_input) return fail(ORR_ERR_NONFINITE, "non-finite position or mass, or negative mass, in the input");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_check(const orr_tree *tree) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    DevParams prm;
    orr_status st = read_params(tree, &prm);
    if (st != ORR_OK) return st;
    if (prm.bad_input) return fail(ORR_ERR_NONFINITE, "non-finite position or mass, or negative mass, in the input");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_export(const orr_tree *tree, uint64_t *keys_sorted, uint32_t *perm, uint8_t *level,
                           uint32_t *begin, uint32_t *count, uint32_t *escape, float *geom, float *s2) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    const Workspace &ws = tree->ws;
    hipStream_t s = tree->stream;
    hipError_t e;
    const size_t n = (size_t)ws.n;
    if (keys_sorted &&
        (e = hipMemcpyAsync(keys_sorted, ws.keys[0], n * 8, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail(e, "export keys");
    if (perm && (e = hipMemcpyAsync(perm, ws.vals[0], n * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail(e, "export perm");
    if (level || begin || count || escape || geom || s2) {
        DevParams prm;
        orr_status st = read_params(tree, &prm);
        if (st != ORR_OK) return st;
        const size_t nn = prm.n_nodes;
        if (level && (e = hipMemcpyAsync(level, ws.level, nn, hipMemcpyDeviceToDevice, s)) != hipSuccess)
            return hip_fail(e, "export level");
        // node records are (com, M | escape, begin, count, s2 bits): strided copies
        const char *rec = reinterpret_cast<const char *>(ws.nodes);
        if (geom && (e = hipMemcpy2DAsync(geom, 16, rec, sizeof(NodeRec), 16, nn, hipMemcpyDeviceToDevice, s)) !=
                        hipSuccess)
            return hip_fail(e, "export geom");
        struct Field {
            void *dst;
            size_t off;
        } fields[4] = {{escape, 16}, {begin, 20}, {count, 24}, {s2, 28}};
        for (const Field &f : fields) {
            if (!f.dst) continue;
            e = hipMemcpy2DAsync(f.dst, 4, rec + f.off, sizeof(NodeRec), 4, nn, hipMemcpyDeviceToDevice, s);
            if (e != hipSuccess) return hip_fail(e, "export topology");
        }
    }
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_tree_export_schedule(const orr_tree *tree, uint32_t *wave_cost, uint32_t *order) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!tree) return fail(ORR_ERR_INVALID_ARG, "tree must not be NULL");
    const Workspace &ws = tree->ws;
    hipError_t e;
    if (wave_cost && (e = hipMemcpyAsync(wave_cost, ws.wave_cost, sizeof(uint32_t) * (size_t)ws.n_waves,
                                         hipMemcpyDeviceToDevice, tree->stream)) != hipSuccess)
        return hip_fail(e, "export wave costs");
    if (order && (e = hipMemcpyAsync(order, ws.wave_order, sizeof(uint32_t) * (size_t)schedule_slots(ws.n_waves),
                                     hipMemcpyDeviceToDevice, tree->stream)) != hipSuccess)
        return hip_fail(e, "export schedule");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_direct_forces(const float *pos, const float *mass, int64_t n, float eps, float *acc,
                             void *hip_stream) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!pos || !mass || !acc) return fail(ORR_ERR_INVALID_ARG, "pos, mass and acc must not be NULL");
    if (n < 1 || n > ORR_MAX_N) return fail(ORR_ERR_RANGE, "n = %lld is outside [1, %lld]", (long long)n, ORR_MAX_N);
    if (check_eps(eps) != ORR_OK) return ORR_ERR_RANGE;
    hipError_t e = maybe_fault("direct");
    if (e == hipSuccess)
        e = launch_direct(pos, mass, n, eps * eps, nullptr, n, acc, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "direct sum");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_direct_forces_targets(const float *pos, const float *mass, int64_t n, float eps, const int64_t *targets,
                                     int64_t n_targets, float *acc, void *hip_stream) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!pos || !mass || !acc || !targets)
        return fail(ORR_ERR_INVALID_ARG, "pos, mass, targets and acc must not be NULL");
    if (n < 1 || n > ORR_MAX_N) return fail(ORR_ERR_RANGE, "n = %lld is outside [1, %lld]", (long long)n, ORR_MAX_N);
    if (n_targets < 0 || n_targets > ORR_MAX_N)
        return fail(ORR_ERR_RANGE, "n_targets = %lld is outside [0, %lld]", (long long)n_targets, ORR_MAX_N);
    if (check_eps(eps) != ORR_OK) return ORR_ERR_RANGE;
    if (n_targets == 0) return ORR_OK;
    hipError_t e = maybe_fault("direct");
    if (e == hipSuccess)
        e = launch_direct(pos, mass, n, eps * eps, targets, n_targets, acc,
                          static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "direct sum over targets");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_direct_forces_fp64_targets(const float *pos, const float *mass, int64_t n, double eps,
                                          const int64_t *targets, int64_t n_targets, double *acc, void *hip_stream) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!pos || !mass || !acc || !targets)
        return fail(ORR_ERR_INVALID_ARG, "pos, mass, targets and acc must not be NULL");
    if (n < 1 || n > ORR_MAX_N) return fail(ORR_ERR_RANGE, "n = %lld is outside [1, %lld]", (long long)n, ORR_MAX_N);
    if (n_targets < 0 || n_targets > ORR_MAX_N)
        return fail(ORR_ERR_RANGE, "n_targets = %lld is outside [0, %lld]", (long long)n_targets, ORR_MAX_N);
    if (!(std::isfinite(eps) && eps >= 0.0))
        return fail(ORR_ERR_RANGE, "eps must be finite and >= 0 (got %g)", eps);
    if (n_targets == 0) return ORR_OK;
    hipError_t e = maybe_fault("direct");
    if (e == hipSuccess)
        e = launch_direct_fp64(pos, mass, n, eps, targets, n_targets, acc,
                               static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "float64 direct sum over targets");
    return ORR_OK;
    ORR_GUARD_END
}

orr_status orr_selftest_inv_sqrt(uint32_t first_bits, uint32_t last_bits, uint64_t *mismatches,
                                 uint32_t *examples, void *hip_stream) {
    ORR_GUARD_BEGIN
    g_last_error.clear();
    if (!mismatches || !examples) return fail(ORR_ERR_INVALID_ARG, "mismatches and examples must not be NULL");
    if (first_bits > last_bits) return fail(ORR_ERR_INVALID_ARG, "first_bits > last_bits");
    hipError_t e = launch_selftest_inv_sqrt(first_bits, (uint64_t)last_bits - first_bits + 1,
                                            reinterpret_cast<unsigned long long *>(mismatches), examples,
                                            static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "inverse square root self-check");
    return ORR_OK;
    ORR_GUARD_END
}

void orr_tree_free(orr_tree *tree) { delete tree; }

}  // extern "C"
