// Schedule of the coherent walk: the order in which its target waves start.
// Computed during the tree build (the costs by k_tree_count, the order by
// eight blocks of the build's last kernel), read by the walk.
#pragma once

#include "orr_internal.h"
#include "walk_common.h"

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
// Waves at the end of a long list that run longest first (see wave_order_list).
constexpr uint32_t kScheduleTail = 1024;
// Slots of the schedule buffer for n_waves waves: the 8 lists and their lengths.
inline int64_t schedule_slots(int64_t n_waves) {
    return (int64_t)kScheduleRegions * ((n_waves + kScheduleRegions - 1) / kScheduleRegions) + 8;
}
static_assert(64 * kMaxLevel + 32 * kMaxLevel < kWaveCostBins, "wave cost range");

// The schedule as 8 lists, one per XCD (the walk's block b runs on XCD b mod 8
// and takes its waves from list b mod 8, in block order), each built by a
// block of its own. The waves are cut into kScheduleRegions contiguous
// regions of R = ceil(n_waves / kScheduleRegions) waves (neighbouring
// targets, whose walks share nodes and leaves in the XCD's L2), and every
// list gets kScheduleRegions / 8 of them: the eighth of the Morton order that
// holds them when the eighths carry nearly equal work, else regions dealt in
// a snake over their total cost (ranks 0..7 to lists 0..7, ranks 8..15 to
// lists 7..0, ...), which evens the work out. List x is stored at
// order[x L .. x L + len_x) with L = R kScheduleRegions / 8; len_x at
// order[8 L + x]. A list of at most 2 kScheduleTail waves (two rounds of an
// XCD's wave slots or fewer) runs in decreasing cost (longest first). A
// longer one runs many rounds, and there the waves that run together should
// be neighbours, which share nodes and leaves in the XCD's L2: its
// kScheduleTail cheapest waves (whole cost bins, so at least that many) end the
// list, longest first, and the others run before them in the list's own
// order (increasing wave index within each region). Equal costs in the tail
// keep the LDS atomics' order, in which neighbouring waves stay together.
constexpr int kOrderCached = 16;  // costs per thread held in registers (list positions t + 1024 i)
constexpr int kRegionUnroll = 4;  // loads in flight per region in the region sums

// floor(w / R) for w < 2^31: with m = floor((2^32 - 1) / R) + 1 (R >= 2) the
// high word of w m is floor(w / R) or one more (w m / 2^32 exceeds w / R by
// less than w / 2^32 < 1/2); one test corrects it. R = 1: w.
__device__ __forceinline__ uint32_t region_of(uint32_t w, uint32_t R, uint32_t m) {
    if (R == 1u) return w;
    uint32_t r = __umulhi(w, m);
    if (r * R > w) r -= 1u;
    return r;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Builds list x. Every block of the schedule sums all regions (the choice of
// lists needs them all), then counting-sorts its own list's waves.
__device__ __forceinline__ void wave_order_list(const uint32_t *__restrict__ cost, uint32_t n_waves,
                                                uint32_t *__restrict__ order, uint32_t x) {
    constexpr uint32_t kBins = kWaveCostBins, kPerList = kScheduleRegions / 8u;
    constexpr uint32_t kWaves = kWaveOrderThreads / 64u;
    __shared__ uint32_t bins[kBins];
    __shared__ uint32_t rcost[kScheduleRegions];
    __shared__ uint32_t myreg[kPerList];
    __shared__ uint32_t wsum[kWaves];
    __shared__ uint32_t head_at[kOrderCached * kWaves];  // head positions of a chunk's (i, wave) groups
    __shared__ uint32_t tail_bin, head_len;
    const uint32_t t = threadIdx.x, lane = t & 63u, wv = t >> 6;
    const uint32_t R = (n_waves + kScheduleRegions - 1u) / kScheduleRegions;
    const uint32_t Rm = R > 1u ? 0xffffffffu / R + 1u : 0u;
    const uint32_t L = kPerList * R;
    auto clamp = [](uint32_t c) { return min(c, kBins - 1u); };

    // Region sums: wave v sums regions v, v + 16, v + 32, v + 48 together.
    {
        constexpr uint32_t kRegs = kScheduleRegions / kWaves;
        uint32_t acc[kRegs] = {};
        for (uint32_t o = lane; o < R; o += 64u * kRegionUnroll) {
#pragma unroll
            for (uint32_t q = 0; q < kRegs; q++) {
                const uint32_t r = wv + q * kWaves;
#pragma unroll
                for (int u = 0; u < kRegionUnroll; u++) {
                    const uint32_t off = o + 64u * (uint32_t)u, w = r * R + off;
                    if (off < R && w < n_waves) acc[q] += clamp(cost[w]);
                }
            }
        }
#pragma unroll
        for (uint32_t q = 0; q < kRegs; q++) {
            const uint32_t v = wave_sum_u32(acc[q]);
            if (lane == 0u) rcost[wv + q * kWaves] = v;
        }
    }
    for (uint32_t b = t; b < kBins; b += kWaveOrderThreads) bins[b] = 0u;
    if (t == 0u) {
        tail_bin = 0u;  // no head unless the bin holding position len - kScheduleTail says otherwise
        head_len = 0u;
    }
    __syncthreads();
    if (wv == 0u) {
        // Contiguous lists (list x = regions 8x .. 8x + 7) when their estimated
        // work is within kContiguousSlack percent of the mean, else a snake
        // over the regions' cost ranks. Wave 0 holds region r in lane r.
        uint64_t tot = 0, mx = 0;
        for (uint32_t y = 0; y < 8u; y++) {
            uint64_t lc = 0;
            for (uint32_t r = 0; r < kPerList; r++) lc += rcost[y * kPerList + r];
            tot += lc;
            mx = lc > mx ? lc : mx;
        }
        uint32_t list;
        if (mx * 800u <= tot * (100u + kContiguousSlack)) {
            list = lane / kPerList;
        } else {
            const uint32_t mine = rcost[lane];
            uint32_t rank = 0;
            for (uint32_t k = 0; k < kScheduleRegions; k++) {
                const uint32_t o = rcost[k];
                rank += (o > mine || (o == mine && k < lane)) ? 1u : 0u;
            }
            const uint32_t round = rank / 8u, pos = rank % 8u;
            list = (round & 1u) ? 7u - pos : pos;
        }
        // this list's regions in increasing order (8 of them in both cases)
        const uint64_t sel = __builtin_amdgcn_ballot_w64(list == x);
        if (list == x) myreg[__builtin_popcountll(sel & ((1ull << lane) - 1ull))] = lane;
    }
    __syncthreads();
    // List position j (0 <= j < L) is wave myreg[j / R] R + j mod R, past
    // n_waves: none. Thread t takes positions t + 1024 i, so one wave
    // instruction covers 64 neighbouring waves.
    auto wave_at = [&](uint32_t j) {
        const uint32_t k = region_of(j, R, Rm);
        return myreg[k] * R + (j - k * R);
    };
    constexpr uint32_t kChunk = kOrderCached * kWaveOrderThreads;
    uint32_t cb[kOrderCached];  // costs of this thread's first kOrderCached positions
    auto load_chunk = [&](uint32_t base, uint32_t(&c)[kOrderCached]) {
#pragma unroll
        for (int i = 0; i < kOrderCached; i++) {
            const uint32_t j = base + t + (uint32_t)i * kWaveOrderThreads, w = j < L ? wave_at(j) : n_waves;
            c[i] = w < n_waves ? clamp(cost[w]) : kBins;  // kBins: no wave
        }
    };
    auto count_chunk = [&](const uint32_t(&c)[kOrderCached]) {
#pragma unroll
        for (int i = 0; i < kOrderCached; i++)
            if (c[i] < kBins) atomicAdd(&bins[kBins - 1u - c[i]], 1u);
    };
    // Places a chunk: a wave of bin b < tail_bin goes to the head, at its
    // rank among the head's waves in list order (position base + 1024 i +
    // 64 v + lane: ranks from the ballots of the chunk's (i, v) groups, scanned
    // in that order by wave 0, plus the head waves of earlier chunks); any
    // other wave to its bin's next place.
    auto place_chunk = [&](uint32_t base, const uint32_t(&c)[kOrderCached]) {
        const uint32_t tb = tail_bin;
        uint64_t head[kOrderCached];
#pragma unroll
        for (int i = 0; i < kOrderCached; i++) {
            head[i] = __builtin_amdgcn_ballot_w64(c[i] < kBins && kBins - 1u - c[i] < tb);
            if (lane == 0u) head_at[i * kWaves + wv] = (uint32_t)__builtin_popcountll(head[i]);
        }
        __syncthreads();
        if (wv == 0u) {
            static_assert(kOrderCached * kWaves == 4u * 64u, "four groups per lane");
            uint32_t g[4], sum = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                g[k] = head_at[4u * lane + k];
                sum += g[k];
            }
            uint32_t inc = sum;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(inc, o, 64);
                if (lane >= (uint32_t)o) inc += y;
            }
            uint32_t at = head_len + inc - sum;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                head_at[4u * lane + k] = at;
                at += g[k];
            }
            if (lane == 63u) head_len = at;
        }
        __syncthreads();
        const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
        for (int i = 0; i < kOrderCached; i++) {
            if (c[i] >= kBins) continue;
            const uint32_t w = wave_at(base + t + (uint32_t)i * kWaveOrderThreads);
            if ((head[i] >> lane) & 1ull)
                order[x * L + head_at[i * kWaves + wv] + (uint32_t)__builtin_popcountll(head[i] & below)] = w;
            else
                order[atomicAdd(&bins[kBins - 1u - c[i]], 1u)] = w;
        }
        __syncthreads();  // head_at is rewritten by the next chunk
    };
    load_chunk(0u, cb);
    count_chunk(cb);
    for (uint32_t base = kChunk; base < L; base += kChunk) {
        uint32_t cx[kOrderCached];
        load_chunk(base, cx);
        count_chunk(cx);
    }
    __syncthreads();
    // Exclusive scan of the bins from x L: thread t owns bins 2t and 2t + 1.
    static_assert(kBins == 2u * kWaveOrderThreads, "two bins per thread");
    const uint32_t c0 = bins[2u * t], c1 = bins[2u * t + 1u];
    uint32_t inc = c0 + c1;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= (uint32_t)o) inc += y;
    }
    if (lane == 63u) wsum[wv] = inc;
    __syncthreads();
    uint32_t before = x * L + inc - c0 - c1;
    for (uint32_t v = 0; v < wv; v++) before += wsum[v];
    bins[2u * t] = before;
    bins[2u * t + 1u] = before + c0;
    // The tail: the bins from the one holding decreasing-cost position
    // len - kScheduleTail on (none of them in a list of at most 2 kScheduleTail).
    {
        uint32_t len = 0;
        for (uint32_t k = 0; k < kPerList; k++) len += min(R, n_waves - min(n_waves, myreg[k] * R));
        const uint32_t h = len > 2u * kScheduleTail ? len - kScheduleTail : 0u;
        const uint32_t s0 = before - x * L, s1 = s0 + c0;  // list positions of bins 2t and 2t + 1
        if (h != 0u && c0 != 0u && s0 <= h && h < s1) tail_bin = 2u * t;
        if (h != 0u && c1 != 0u && s1 <= h && h < s1 + c1) tail_bin = 2u * t + 1u;
    }
    __syncthreads();
    place_chunk(0u, cb);
    for (uint32_t base = kChunk; base < L; base += kChunk) {
        uint32_t cx[kOrderCached];
        load_chunk(base, cx);
        place_chunk(base, cx);
    }
    if (t == 0u) {
        uint32_t len = 0;
        for (uint32_t k = 0; k < kPerList; k++) len += min(R, n_waves - min(n_waves, myreg[k] * R));
        order[8u * L + x] = len;
    }
}

// Sorted targets of this lane's target wave: block b runs on XCD b mod 8 and
// takes its target waves from that XCD's list of the schedule, in block order
// (slot s of the XCD runs list entry s: targets 64 (wave0 + w) .. + 63 of the
// schedule's wave w, whose waves start at wave0). With kSplit hardware waves
// per target wave, consecutive hardware waves of the XCD share one slot and
// *part receives this wave's share (0 .. kSplit - 1). Slots past the list get
// the first target past the schedule's waves, which no lane walks.
template <uint32_t kSplit>
__device__ __forceinline__ uint32_t scheduled_target(const uint32_t *__restrict__ order, uint32_t n_waves,
                                                     uint32_t wave0, uint32_t *part) {
    const uint32_t L = (kScheduleRegions / 8u) * ((n_waves + kScheduleRegions - 1u) / kScheduleRegions);
    const uint32_t x = blockIdx.x & 7u;
    // The hardware waves of XCD x in launch order; kSplit consecutive ones
    // share one target wave (a work-group holds 4 waves; teams of 8 or 16
    // span 2 or 4 work-groups, which need not run together).
    const uint32_t hw = (blockIdx.x >> 3) * (kWalkBlock / 64u) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t s = hw / kSplit;
    *part = hw % kSplit;
    const uint32_t w = s < order[8u * L + x] ? min(order[x * L + s], n_waves) : n_waves;
    return (wave0 + w) * 64u + (threadIdx.x & 63u);
}

}  // namespace orr
