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
// Slots of the schedule buffer for n_waves waves: the 8 lists and their lengths.
inline int64_t schedule_slots(int64_t n_waves) {
    return (int64_t)kScheduleRegions * ((n_waves + kScheduleRegions - 1) / kScheduleRegions) + 8;
}
static_assert(64 * kMaxLevel + 32 * kMaxLevel < kWaveCostBins, "wave cost range");

// One block: the schedule as 8 lists, one per XCD (the walk's block b runs on
// XCD b mod 8 and takes its waves from list b mod 8, in block order). The
// waves are cut into kScheduleRegions contiguous regions of R =
// ceil(n_waves / kScheduleRegions) waves (neighbouring targets, whose walks
// share nodes and leaves in the XCD's L2); the regions are dealt to the lists
// in a snake over their total cost (ranks 0..7 to lists 0..7, ranks 8..15 to
// lists 7..0, ...), so every list gets kScheduleRegions / 8 regions and
// nearly the same work. List x is stored at order[x L .. x L + len_x) with L =
// R kScheduleRegions / 8, its waves in decreasing cost (longest first);
// len_x at order[8 L + x]. Equal costs keep the LDS atomics' order.
constexpr uint32_t kOrderSlots = 8u * kWaveCostBins;
__device__ __forceinline__ void wave_order_block(const uint32_t *__restrict__ cost, uint32_t n_waves,
                                                 uint32_t *__restrict__ order) {
    __shared__ uint32_t slots[kOrderSlots];
    __shared__ uint32_t wsum[kWaveOrderThreads / 64];
    __shared__ uint32_t rcost[kScheduleRegions];
    __shared__ uint32_t rlist[kScheduleRegions];
    const uint32_t t = threadIdx.x, lane = t & 63u, wv = t >> 6;
    const uint32_t R = (n_waves + kScheduleRegions - 1u) / kScheduleRegions;
    for (uint32_t b = t; b < kOrderSlots; b += kWaveOrderThreads) slots[b] = 0u;
    if (t < kScheduleRegions) rcost[t] = 0u;
    __syncthreads();
    for (uint32_t w = t; w < n_waves; w += kWaveOrderThreads) atomicAdd(&rcost[w / R], cost[w]);
    __syncthreads();
    if (t < kScheduleRegions) {  // rank by decreasing cost (ties by index), snake over the 8 lists
        const uint32_t mine = rcost[t];
        uint32_t rank = 0;
        for (uint32_t k = 0; k < kScheduleRegions; k++) {
            const uint32_t o = rcost[k];
            rank += (o > mine || (o == mine && k < t)) ? 1u : 0u;
        }
        const uint32_t round = rank / 8u, pos = rank % 8u;
        rlist[t] = (round & 1u) ? 7u - pos : pos;
    }
    __syncthreads();
    auto slot_of = [&](uint32_t w) {
        const uint32_t c = min(cost[w], (uint32_t)kWaveCostBins - 1u);
        return rlist[w / R] * (uint32_t)kWaveCostBins + ((uint32_t)kWaveCostBins - 1u - c);
    };
    for (uint32_t w = t; w < n_waves; w += kWaveOrderThreads) atomicAdd(&slots[slot_of(w)], 1u);
    __syncthreads();
    // list x's segment starts at x L: scan each list's 2048 bins separately.
    // 8 lists x 2048 bins; thread t owns list t / 128, bins 16 (t % 128) .. + 15.
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
    for (uint32_t w = t; w < n_waves; w += kWaveOrderThreads) order[atomicAdd(&slots[slot_of(w)], 1u)] = w;
    // list lengths for the walk, after the 8 list segments: order[8 L + x]
    if (t < 8u) {
        uint32_t len = 0;
        for (uint32_t r = 0; r < kScheduleRegions; r++)
            if (rlist[r] == t) len += min(R, n_waves - min(n_waves, r * R));
        order[8u * L + t] = len;
    }
}

}  // namespace orr
