// Internal declarations of liborr: workspace layout, device-side parameter
// block, kernel launch wrappers. Not part of the public ABI (include/orr.h).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace orr {

constexpr int kMaxLevel = 21;            // 21 bits per axis, 63-bit keys
constexpr uint32_t kQMax = 2097151u;     // 2^21 - 1
constexpr uint32_t kNoParent = 0xffffffffu;

// Sort tiles: 512 threads x 2, 4 or 8 keys. Small inputs take small tiles:
// a pass over few tiles is bound by each tile's latency, which shrinks with
// the keys per thread, while large inputs gain from the fewer tiles (and
// shorter look-back) of large ones.
constexpr int kTileThreads = 512;
inline int sort_tile_items(int64_t n) { return n <= 32768 ? 2 : n <= 262144 ? 4 : 8; }
inline int64_t sort_tile_keys(int64_t n) { return (int64_t)kTileThreads * sort_tile_items(n); }
constexpr int kRadixBits = 8;
constexpr int kRadixBins = 1 << kRadixBits;
// The main sort orders the keys by their high 32 bits (bits 31..62) in 4
// passes; runs of equal high bits are then ordered by the low 31 bits in
// place (k_sort_fix). Runs longer than kFixMaxRun go to the fallback, which
// sorts their elements together by (rank of the run, low 31 bits) when there
// are at most kMaxLongRuns of them, and the whole array by the full key
// otherwise.
constexpr int kRadixPasses = 4;
constexpr int kSortLowBits = 31;
constexpr int kFullPasses = 8;           // 64 / 8; bit 63 is always zero
constexpr int kRunPasses = 5;            // digits of (run rank < 64) << 31 | low bits
constexpr int kFixThreads = 512;         // positions per block of the run fix-up
constexpr int kFixHalo = 64;             // window margin: runs up to 64 are finished per thread
constexpr int kFixMaxRun = 4096;         // longest run finished by one work-group
constexpr int kMaxLongRuns = 64;         // longer runs the fallback sorts by themselves
constexpr int kFallbackBlocks = 512;     // persistent blocks of the fallback sort
// The fallback's scratch in hist_part (free after k_digit_offsets): digit
// counts, then the list of long runs (first position, end) as uint2.
constexpr int kFbHistWords = kFullPasses * kRadixBins;
constexpr int kFbListWords = 2 * kMaxLongRuns;

constexpr int kCubeBlocks = 256;         // partial blocks of the root-cube reduction

constexpr int kSortHistBlocks = 256;     // blocks of the key + histogram pass
static_assert(kFbHistWords + kFbListWords <= kSortHistBlocks * kRadixPasses * kRadixBins, "fallback scratch fits");
constexpr uint32_t kCutParticles = 4096; // subtrees of at most this many particles get one workgroup
constexpr int kWaveCostBins = 2048;      // bins of the walk schedule's wave cost

// Device-resident scalars of one build, at the start of the workspace.
struct DevParams {
    float lo[3];
    float side;
    float scale;          // 2^21 / side
    uint32_t bad_input;   // bit 0: non-finite position/mass, negative mass or overflowing extent;
                          // bit 1: a look-back or phase wait of the sort gave up (never expected);
                          // bit 2 (kBadIndex): an index check of the checked build failed
    uint32_t n_nodes;
    uint32_t n_leaves;    // filled by the info kernels only
    uint32_t depth;
    uint32_t max_leaf_count;
    uint32_t sort_ticket[kRadixPasses];  // tile tickets of the one-sweep passes
    uint32_t n_cut;                      // entries of the cut-node list
    uint32_t n_top;                      // entries of the above-the-cut list
    uint32_t sort_fallback;              // set by k_sort_fix: some run is longer than kFixMaxRun
    uint32_t n_long;                     // such runs (listed up to kMaxLongRuns)
    uint32_t fb_ticket;                  // work tickets of the fallback sort
    uint32_t fb_hist_done;               // finished tiles of the fallback's histogram phase
    uint32_t fb_plan;                    // bit q: the fallback's digit q is not the same for all keys
    uint32_t fb_done[1 + kFullPasses];   // phase 0 (nt once the plan is set) and finished tiles per pass
    uint32_t n_particles;                // particles of the build
    uint32_t pad;
};
constexpr uint32_t kBadIndex = 4u;       // bit of DevParams::bad_input
static_assert(sizeof(DevParams) == 128, "DevParams layout");

// One tree node, 32 bytes: g = (com.x, com.y, com.z, M),
// t = (escape, begin, count, bits of s^2). A wave reads it with one scalar load.
struct alignas(32) NodeRec {
    float4 g;
    uint4 t;
};
static_assert(sizeof(NodeRec) == 32, "NodeRec layout");

// Device pointers carved from the caller's workspace.
struct Workspace {
    DevParams *prm;
    float *cube_part;      // [kCubeBlocks][8]
    uint64_t *keys[2];     // [n] radix ping-pong: the passes start and end in keys[1], the
                           // run fix-up writes the sorted keys to keys[0]
    uint32_t *vals[2];     // [n] payload: original index; perm ends in vals[0]
    uint32_t *hist_part;   // [kSortHistBlocks][kRadixPasses][kRadixBins] digit counts per block;
                           // after the digit offsets, the fallback's counts and list of long runs
    uint32_t *digit_offs;  // [kRadixPasses][kRadixBins] first output slot of each digit
    uint64_t *lb_words;    // look-back words of the sort's passes (room for the fallback's 8)
    int64_t n_lb_words;
    float4 *xs;            // [n] sorted (x, y, z, m)
    uint32_t *info;        // [n] first level started | leaf depth << 8
    uint32_t *base;        // [n + 1] nodes started by earlier particles of the same 256-particle tile
    uint32_t *tile_sum;    // [tiles + 1] nodes started per 256-particle tile, then their exclusive scan
    NodeRec *nodes;        // [max_nodes]
    float4 *msum;          // [max_nodes >= n] (S, M), unnormalised sums for the parent; before the
                           // build, the input particles as float4 for the sort's gather
    uint8_t *level;        // [max_nodes]
    uint32_t *cut_list;    // [max_nodes] roots of the subtrees finished by one workgroup each
    uint32_t *top_list;    // [max_top] nodes above the cut
    uint32_t *kids;        // [9 max_top] child count and children of each node above the cut
    uint32_t *wave_cost;   // [n_waves] estimated run time of a wave of 64 sorted targets
    uint32_t *wave_order;  // walk schedule: 8 XCD lists of target waves by decreasing cost, their lengths
    uint32_t *range_order;  // the same for the waves of one target range (range walks)
    int64_t n_waves;       // ceil(n / 64)
    int64_t max_top;
    int64_t n;
    int32_t leaf_cap;
    int64_t max_nodes;
    int64_t n_tiles;       // sort tiles of kTile keys
};

inline int64_t max_nodes_for(int64_t n, int32_t leaf_cap) {
    return n + 21 * (n / (leaf_cap + 1)) + 1;
}

// Nodes holding more than kCutParticles are disjoint on each of the 22 levels.
inline int64_t max_top_for(int64_t n) { return 22 * (n / (kCutParticles + 1)) + 1; }

// Lays the workspace out from `base` (which may be null for sizing) and
// returns the bytes it needs.
size_t carve_workspace(void *base, int64_t n, int32_t leaf_cap, Workspace *ws);

// ---- launch wrappers (each returns hipGetLastError() of its launches) ----
hipError_t launch_cube(const float *pos, const float *mass, const Workspace &ws, hipStream_t s);
// Keys, digit histograms, the 4 high-bit passes, the run fix-up with the
// gather, and the fallback (which returns at once unless the fix-up asked for
// it); after_keys (may be null) is recorded between the key pass and the
// first sort pass.
hipError_t launch_keys_and_sort(const float *pos, const float *mass, const Workspace &ws, hipStream_t s,
                                hipEvent_t after_keys);
hipError_t launch_build(const Workspace &ws, hipStream_t s);
hipError_t launch_moments(const Workspace &ws, hipStream_t s);
hipError_t launch_tree_info(const Workspace &ws, hipStream_t s);
// Walk kinds: the independent walk, the coherent walk (ballot advance), the
// coherent walk advancing by an explicit wave minimum (same results).
enum { kWalkIndependent = 0, kWalkCoherent = 1, kWalkCoherentMin = 2 };
hipError_t launch_walk(const Workspace &ws, int mode, float eps2, float theta2, float *acc,
                       uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                       hipStream_t s);
// Sorted targets [first, first + count) of whole waves (first a multiple of
// 64; count too unless the range ends at n); order: the coherent walk's
// schedule of the range's waves (ws.wave_order for all targets, else
// ws.range_order after launch_range_schedule).
struct WalkRange {
    int64_t first, count;
    const uint32_t *order;
};
hipError_t launch_walk_range(const Workspace &ws, int mode, const WalkRange &rg, float eps2, float theta2,
                             float *acc, uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp,
                             uint32_t *n_pc, hipStream_t s);
// The walk schedule of waves [wave0, wave0 + n_waves) into ws.range_order.
hipError_t launch_range_schedule(const Workspace &ws, int64_t wave0, int64_t n_waves, hipStream_t s);
// Group widths 1, 2, 4, ..., 64 (hipErrorInvalidValue otherwise); descend:
// the descend-together variant.
hipError_t launch_walk_grouped(const Workspace &ws, int width, bool descend, float eps2, float theta2, float *acc,
                               uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                               hipStream_t s);
// The coherent walk at coherence width 32 (two node indices per wave), 64
// (launch_walk), 128 or 256 (2 or 4 waves of a work-group sharing one node
// index); hipErrorInvalidValue for other widths.
hipError_t launch_walk_width(const Workspace &ws, int width, float eps2, float theta2, float *acc,
                             uint32_t *visits_own, uint32_t *visits_stepped, uint32_t *n_pp, uint32_t *n_pc,
                             hipStream_t s);
hipError_t launch_selftest_inv_sqrt(uint32_t first, uint64_t count, unsigned long long *mismatches,
                                    uint32_t *examples, hipStream_t s);
// All-pairs sums for n_out targets: caller indices targets[0 .. n_out) (NaN
// for an index outside [0, n)), or particles 0 .. n_out - 1 (n_out = n) when
// targets is null.
hipError_t launch_direct(const float *pos, const float *mass, int64_t n, float eps2, const int64_t *targets,
                         int64_t n_out, float *acc, hipStream_t s);
// Compensated float64 sums for targets[0 .. n_out) (NaN for an index outside [0, n)).
hipError_t launch_direct_fp64(const float *pos, const float *mass, int64_t n, double eps, const int64_t *targets,
                              int64_t n_out, double *acc, hipStream_t s);
uint32_t morton_hist_blocks(int64_t n);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace orr
