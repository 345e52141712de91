// Schedule of the coherent walk: the order in which its target waves start.
// Computed during the tree build (the costs by k_tree_count, the order by one
// block of the build's last kernel), read by the walk.
#pragma once

#include "orr_internal.h"

namespace orr {

// Walk schedule. How long a wave runs grows with the particle density
// around its targets, which the depth of a target's leaf measures, and with
// how spread out its 64 targets are: the wave steps through the union of
// their walks, which grows when the targets span a large cell. The cost of a
// wave is its summed leaf depth plus 32 times the levels between its deepest
// leaf and the smallest cell holding all its targets (from the common prefix
// of its first and last sorted key); the tree build's k_tree_count writes
// it. Target waves start in order of decreasing cost, so the longest ones
// start first and the last to start are short: longest-first list
// scheduling, which keeps the grid's tail short when a wave runs for a large
// part of the whole launch. The schedule decides only when a wave runs,
// never what it computes.
constexpr int kWaveOrderThreads = kWaveCostBins / 2;
constexpr uint32_t kScheduleRegions = 64;
constexpr uint32_t kContiguousSlack = 5;  // percent
// Slots of the schedule buffer for n_waves waves: the 8 lists and their lengths.
inline int64_t schedule_slots(int64_t n_waves) {
    return (int64_t)kScheduleRegions * ((n_waves + kScheduleRegions - 1) / kScheduleRegions) + 8;
}
static_assert(64 * kMaxLevel + 32 * kMaxLevel < kWaveCostBins, "wave cost range");

// One block: the schedule as 8 lists, one per XCD (the walk's block b runs on
// XCD b mod 8 and takes its waves from list b mod 8, in block order). The
// waves are cut into kScheduleRegions contiguous regions of R =
// ceil(n_waves / kScheduleRegions) waves (neighbouring targets, whose walks
// share nodes and leaves in the XCD's L2), and every list gets
// kScheduleRegions / 8 of them: the eighth of the Morton order that holds
// them when the eighths carry nearly equal work, else regions dealt in a
// snake over their total cost (ranks 0..7 to lists 0..7, ranks 8..15 to lists
// 7..0, ...), which evens the work out. List x is stored at
// order[x L .. x L + len_x) with L = R kScheduleRegions / 8, its waves in
// decreasing cost (longest first); len_x at order[8 L + x]. Equal costs keep
// the LDS atomics' order.
constexpr uint32_t kOrderSlots = 8u * kWaveCostBins;
constexpr int kOrderCached = 16;  // costs per thread held in registers (waves t + 1024 j)

// floor(w / R) for w < 2^31: with m = floor((2^32 - 1) / R) + 1 (R >= 2) the
// high word of w m is floor(w / R) or one more (w m / 2^32 exceeds w / R by
// less than w / 2^32 < 1/2); one test corrects it. R = 1: w.
__device__ __forceinline__ uint32_t region_of(uint32_t w, uint32_t R, uint32_t m) {
    if (R == 1u) return w;
    uint32_t r = __umulhi(w, m);
    if (r * R > w) r -= 1u;
    return r;
}

// Costs of waves base + t + kWaveOrderThreads j (0 past n_waves), clamped to
// the bins, all loads issued together.
__device__ __forceinline__ void load_costs(const uint32_t *__restrict__ cost, uint32_t n_waves, uint32_t base,
                                           uint32_t t, uint32_t (&cb)[kOrderCached]) {
#pragma unroll
    for (int j = 0; j < kOrderCached; j++) {
        const uint32_t w = base + t + (uint32_t)j * kWaveOrderThreads;
        cb[j] = w < n_waves ? min(cost[w], (uint32_t)kWaveCostBins - 1u) : 0u;
    }
}

__device__ __forceinline__ void wave_order_block(const uint32_t *__restrict__ cost, uint32_t n_waves,
                                                 uint32_t *__restrict__ order) {
    __shared__ uint32_t slots[kOrderSlots];
    __shared__ uint32_t wsum[kWaveOrderThreads / 64];
    __shared__ uint32_t rcost[kScheduleRegions];
    __shared__ uint32_t rlist[kScheduleRegions];
    const uint32_t t = threadIdx.x, lane = t & 63u, wv = t >> 6;
    const uint32_t R = (n_waves + kScheduleRegions - 1u) / kScheduleRegions;
    const uint32_t Rm = R > 1u ? 0xffffffffu / R + 1u : 0u;
    constexpr uint32_t kChunk = kOrderCached * kWaveOrderThreads;  // waves per pass over the threads
    uint32_t cb[kOrderCached];  // costs of waves t + j kWaveOrderThreads, kept for every pass
    load_costs(cost, n_waves, 0u, t, cb);
    for (uint32_t b = t; b < kOrderSlots; b += kWaveOrderThreads) slots[b] = 0u;
    if (t < kScheduleRegions) rcost[t] = 0u;
    __syncthreads();
    // Region sums. The 64 lanes of a wave hold 64 neighbouring waves, mostly
    // of one region: then one lane adds their sum. Called by whole waves.
    auto add_region = [&](uint32_t w, uint32_t c) {
        const bool in = w < n_waves;
        const uint32_t r = in ? region_of(w, R, Rm) : 0u;
        const uint32_t r0 = __builtin_amdgcn_readfirstlane(r);
        if (__builtin_amdgcn_ballot_w64(in && r == r0) == __builtin_amdgcn_ballot_w64(true)) {
            uint32_t v = in ? c : 0u;
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
            if (lane == 0u) atomicAdd(&rcost[r0], v);
        } else if (in) {
            atomicAdd(&rcost[r], c);
        }
    };
#pragma unroll
    for (int j = 0; j < kOrderCached; j++) add_region(t + (uint32_t)j * kWaveOrderThreads, cb[j]);
    for (uint32_t base = kChunk; base < n_waves; base += kChunk) {  // more waves: a chunk at a time
        uint32_t cx[kOrderCached];
        load_costs(cost, n_waves, base, t, cx);
#pragma unroll
        for (int j = 0; j < kOrderCached; j++) add_region(base + t + (uint32_t)j * kWaveOrderThreads, cx[j]);
    }
    __syncthreads();
    if (t < kScheduleRegions) {
        // Contiguous lists (list x = regions 8x .. 8x + 7, each XCD one eighth
        // of the Morton order) when their estimated work is within
        // kContiguousSlack percent of the mean, else a snake over the regions'
        // cost ranks.
        uint64_t tot = 0, mx = 0;
        for (uint32_t x = 0; x < 8u; x++) {
            uint64_t lc = 0;
            for (uint32_t r = 0; r < kScheduleRegions / 8u; r++) lc += rcost[x * (kScheduleRegions / 8u) + r];
            tot += lc;
            mx = lc > mx ? lc : mx;
        }
        if (mx * 800u <= tot * (100u + kContiguousSlack)) {
            rlist[t] = t / (kScheduleRegions / 8u);
        } else {
            const uint32_t mine = rcost[t];
            uint32_t rank = 0;
            for (uint32_t k = 0; k < kScheduleRegions; k++) {
                const uint32_t o = rcost[k];
                rank += (o > mine || (o == mine && k < t)) ? 1u : 0u;
            }
            const uint32_t round = rank / 8u, pos = rank % 8u;
            rlist[t] = (round & 1u) ? 7u - pos : pos;
        }
    }
    __syncthreads();
    auto slot_of = [&](uint32_t w, uint32_t c) {
        return rlist[region_of(w, R, Rm)] * (uint32_t)kWaveCostBins + ((uint32_t)kWaveCostBins - 1u - c);
    };
    auto count_chunk = [&](uint32_t base, const uint32_t(&c)[kOrderCached]) {
#pragma unroll
        for (int j = 0; j < kOrderCached; j++) {
            const uint32_t w = base + t + (uint32_t)j * kWaveOrderThreads;
            if (w < n_waves) atomicAdd(&slots[slot_of(w, c[j])], 1u);
        }
    };
    count_chunk(0u, cb);
    for (uint32_t base = kChunk; base < n_waves; base += kChunk) {
        uint32_t cx[kOrderCached];
        load_costs(cost, n_waves, base, t, cx);
        count_chunk(base, cx);
    }
    __syncthreads();
    // List x's segment starts at x L: each list's 2048 bins are scanned on
    // their own; thread t owns list t / 128, bins 16 (t % 128) .. + 15.
    const uint32_t L = (kScheduleRegions / 8u) * R;
    const uint32_t list = t / 128u, part = t % 128u;
    uint32_t c[16], tot = 0;
#pragma unroll
    for (int k = 0; k < 16; k++) {
        c[k] = slots[list * kWaveCostBins + 16u * part + k];
        tot += c[k];
    }
    uint32_t x = tot;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= (uint32_t)o) x += y;
    }
    if (lane == 63u) wsum[wv] = x;
    __syncthreads();
    uint32_t run = list * L + x - tot;
    if (wv & 1u) run += wsum[wv - 1];  // two waves per list
#pragma unroll
    for (int k = 0; k < 16; k++) {
        slots[list * kWaveCostBins + 16u * part + k] = run;
        run += c[k];
    }
    __syncthreads();
    auto place_chunk = [&](uint32_t base, const uint32_t(&c)[kOrderCached]) {
#pragma unroll
        for (int j = 0; j < kOrderCached; j++) {
            const uint32_t w = base + t + (uint32_t)j * kWaveOrderThreads;
            if (w < n_waves) order[atomicAdd(&slots[slot_of(w, c[j])], 1u)] = w;
        }
    };
    place_chunk(0u, cb);
    for (uint32_t base = kChunk; base < n_waves; base += kChunk) {
        uint32_t cx[kOrderCached];
        load_costs(cost, n_waves, base, t, cx);
        place_chunk(base, cx);
    }
    // list lengths for the walk, after the 8 list segments: order[8 L + x]
    if (t < 8u) {
        uint32_t len = 0;
        for (uint32_t r = 0; r < kScheduleRegions; r++)
            if (rlist[r] == t) len += min(R, n_waves - min(n_waves, r * R));
        order[8u * L + t] = len;
    }
}

}  // namespace orr
