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
static_assert(64 * kMaxLevel + 32 * kMaxLevel < kWaveCostBins, "wave cost range");

// One block: counting sort of the waves by decreasing cost. Waves of equal
// cost may come out in any order; in practice the LDS atomics serve a wave's
// lanes in lane order, which keeps neighbouring waves of equal cost together
// (spreading equal costs over sub-bins to cut atomic conflicts made the
// 8M walk 2 % slower). The first kOrderCached costs of each thread are loaded
// once, all at the start.
constexpr int kOrderCached = 16;

__device__ __forceinline__ void wave_order_block(const uint32_t *__restrict__ cost, uint32_t n_waves,
                                                 uint32_t *__restrict__ order) {
    __shared__ uint32_t bins[kWaveCostBins];
    __shared__ uint32_t wsum[kWaveOrderThreads / 64];
    const uint32_t t = threadIdx.x, lane = t & 63u, wv = t >> 6;
    uint32_t cb[kOrderCached];  // cost bins of waves t + j kWaveOrderThreads
#pragma unroll
    for (int j = 0; j < kOrderCached; j++) {
        const uint32_t w = t + (uint32_t)j * kWaveOrderThreads;
        cb[j] = w < n_waves ? min(cost[w], (uint32_t)kWaveCostBins - 1u) : 0u;
    }
    for (uint32_t b = t; b < (uint32_t)kWaveCostBins; b += kWaveOrderThreads) bins[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kOrderCached; j++)
        if (t + (uint32_t)j * kWaveOrderThreads < n_waves) atomicAdd(&bins[cb[j]], 1u);
    for (uint32_t w = t + kOrderCached * kWaveOrderThreads; w < n_waves; w += kWaveOrderThreads)
        atomicAdd(&bins[min(cost[w], (uint32_t)kWaveCostBins - 1u)], 1u);
    __syncthreads();
    // Exclusive scan in decreasing cost; thread t owns bins b0 = top - 2t and b0 - 1.
    const uint32_t b0 = (uint32_t)kWaveCostBins - 1u - 2u * t, b1 = b0 - 1u;
    const uint32_t c0 = bins[b0], c1 = bins[b1];
    uint32_t x = c0 + c1;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= (uint32_t)o) x += y;
    }
    if (lane == 63u) wsum[wv] = x;
    __syncthreads();
    uint32_t before = 0u;
    for (uint32_t k = 0; k < wv; k++) before += wsum[k];
    const uint32_t excl = before + x - (c0 + c1);
    bins[b0] = excl;
    bins[b1] = excl + c0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kOrderCached; j++) {
        const uint32_t w = t + (uint32_t)j * kWaveOrderThreads;
        if (w < n_waves) order[atomicAdd(&bins[cb[j]], 1u)] = w;
    }
    for (uint32_t w = t + kOrderCached * kWaveOrderThreads; w < n_waves; w += kWaveOrderThreads) {
        const uint32_t pos = atomicAdd(&bins[min(cost[w], (uint32_t)kWaveCostBins - 1u)], 1u);
        order[pos] = w;
    }
}

}  // namespace orr
