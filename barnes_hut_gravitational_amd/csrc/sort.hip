// Morton keys with their digit histograms, and the stable one-sweep LSD radix
// sort of (key, index) with the gather into tree order fused into its last
// pass.
//
// The orrery performance page ("Where one evaluation goes", "The largest
// row") measures the host Morton sort as the largest single cost of an
// evaluation and names a device radix sort as the first thing to do; here it
// runs on the GPU. Equal keys keep ascending original index because every
// pass is stable and the payload starts as the identity.
//
// Pass structure (8 passes of 8-bit digits, bit 63 is always zero):
//   * k_morton_hist computes every key once and the 8 digit histograms of all
//     keys; k_digit_offsets turns them into the first output slot of each
//     digit in each pass.
//   * k_onesweep, one launch per pass: a tile of 512 threads x 2, 4 or 8 keys
//     (by the input's size, sort_tile_items) takes a ticket (its position in the output), counts its digits and
//     publishes the counts at once, ranks its keys stably inside each wave
//     (lanes with the same digit found with 8 ballots), and then adds the
//     counts of the tiles before it by decoupled look-back: walking back over
//     predecessors' published words, four per step, until one carries an
//     inclusive prefix. Publishing before the ranking lets the successors'
//     walks find the counts sooner. Tickets are taken in the order
//     blocks start, so every predecessor is running or done and publishes its
//     counts without waiting on anyone; each wait is nevertheless bounded and
//     reports an error. The tile is then reordered by digit in LDS and
//     written out in that order: each digit's run of the tile lands in one
//     contiguous stretch of the output, stored by consecutive threads.
#include "orr_internal.h"

namespace orr {

namespace {

// Look-back words: high 32 bits = state, low 32 bits = value.
constexpr uint64_t kStAggregate = 1ull << 32;
constexpr uint64_t kStInclusive = 2ull << 32;
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ __forceinline__ uint64_t lb_load(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void lb_store(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#ifndef ORR_LB_WIN
#define ORR_LB_WIN 4
#endif
// Publishes a tile's value for one digit: inclusive for tile 0, else an
// aggregate that successors can add while the tile works on.
__device__ __forceinline__ void lb_publish(uint64_t *words, uint32_t tile, uint32_t stride, uint32_t mine) {
    lb_store(words + (uint64_t)tile * stride, (tile == 0 ? kStInclusive : kStAggregate) | mine);
}

// Exclusive prefix over earlier tiles of one value, after lb_publish: walks
// back over the predecessors' words, ORR_LB_WIN at a time, adding aggregates
// until an inclusive value, then publishes its own inclusive value. Sets
// *err on a wait that never ends.
__device__ __forceinline__ uint32_t lb_resolve(uint64_t *words, uint32_t tile, uint32_t stride, uint32_t mine,
                                               uint32_t *err) {
    if (tile == 0) return 0;
    uint32_t excl = 0, spins = 0;
    int64_t t = (int64_t)tile - 1;
    while (true) {
        uint64_t v[ORR_LB_WIN];
#pragma unroll
        for (int k = 0; k < ORR_LB_WIN; k++)
            v[k] = t - k >= 0 ? lb_load(words + (uint64_t)(t - k) * stride) : kStInclusive;
        int used = 0;
        bool done = false;
#pragma unroll
        for (int k = 0; k < ORR_LB_WIN; k++) {
            if (done || used < k) continue;
            const uint64_t st = v[k] & ~0xffffffffull;
            if (st == kStInclusive) {
                excl += (uint32_t)v[k];
                done = true;
            } else if (st == kStAggregate) {
                excl += (uint32_t)v[k];
                used = k + 1;
            }
        }
        if (done) break;
        if (used == 0 && ++spins > kSpinLimit) {  // a predecessor never published: give up, flagged
            atomicOr(err, 2u);
            break;
        }
        t -= used;
    }
    lb_store(words + (uint64_t)tile * stride, kStInclusive | (excl + mine));
    return excl;
}

// Spread the low 21 bits of v so that bit b lands on bit 3b (mask-and-shift
// bit interleaving).
__device__ __forceinline__ uint64_t spread3(uint32_t v) {
    uint64_t x = v & 0x1fffffu;
    x = (x | (x << 32)) & 0x001f00000000ffffull;
    x = (x | (x << 16)) & 0x001f0000ff0000ffull;
    x = (x | (x << 8)) & 0x100f00f00f00f00full;
    x = (x | (x << 4)) & 0x10c30c30c30c30c3ull;
    x = (x | (x << 2)) & 0x1249249249249249ull;
    return x;
}

// q = min(trunc((x - lo) * scale), 2^21 - 1); anything not >= 0 (only
// possible for flagged input) maps to 0.
__device__ __forceinline__ uint32_t quantise(float x, float lo, float scale) {
    const float t = (x - lo) * scale;
    if (t >= 2097151.0f) return kQMax;
    return t >= 0.0f ? (uint32_t)t : 0u;
}

__device__ __forceinline__ float wave_min(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// The root cube from the per-block partials of k_cube_partial (min x, y, z,
// max x, y, z, flag bits), by one wave: corner lo = the minima (-0 made +0,
// so the corner is unique), side = the largest extent (1 if it is 0 or not
// finite, the latter flagged), scale = 2^21 / side correctly rounded. Every
// block of the key kernel computes the same values from the same partials.
__device__ __forceinline__ void cube_from_partials(const float *__restrict__ part, int nparts, float lo[3],
                                                   float &side, uint32_t &bad) {
    const int lane = threadIdx.x & 63;
    float r[6] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY};
    uint32_t b = 0;
    for (int q = lane; q < nparts; q += 64) {
        for (int k = 0; k < 3; k++) r[k] = fminf(r[k], part[8 * q + k]);
        for (int k = 3; k < 6; k++) r[k] = fmaxf(r[k], part[8 * q + k]);
        b |= __float_as_uint(part[8 * q + 6]);
    }
    for (int k = 0; k < 3; k++) r[k] = wave_min(r[k]);
    for (int k = 3; k < 6; k++) r[k] = wave_max(r[k]);
    bad = __ballot(b != 0) != 0ull;
    side = 0.0f;
    for (int a = 0; a < 3; a++) {
        lo[a] = r[a] + 0.0f;
        const float ext = r[3 + a] - lo[a];
        if (ext > side) side = ext;
    }
    if (!isfinite(side) || !isfinite(lo[0]) || !isfinite(lo[1]) || !isfinite(lo[2])) {
        bad = 1;  // keep the rest of the build well-formed
        side = 1.0f;
        for (int a = 0; a < 3; a++)
            if (!isfinite(lo[a])) lo[a] = 0.0f;
    }
    if (side == 0.0f) side = 1.0f;
}

// Keys and the identity payload; each block's 8 digit histograms to
// part[block][pass][digit]; zeroes the look-back words of the build; copies
// every particle as one float4 (x, y, z, m) in input order to xs0, which the
// last pass gathers from (one aligned load per particle instead of a 12-byte
// and a 4-byte one). Each
// block first forms the root cube from the partials; block 0 also stores it
// in prm with the input flag and resets the build's device counters.
__global__ __launch_bounds__(256) void k_morton_hist(const float *__restrict__ pos, const float *__restrict__ mass,
                                                     float4 *__restrict__ xs0, uint32_t n,
                                                     const float *__restrict__ cube_part, int cube_parts,
                                                     DevParams *__restrict__ prm, uint64_t *__restrict__ keys,
                                                     uint32_t *__restrict__ idx, uint32_t *__restrict__ part,
                                                     uint64_t *__restrict__ lb_words, uint64_t n_lb_words) {
    __shared__ uint32_t h[kRadixPasses * kRadixBins];
    __shared__ float s_cube[4];
    for (int k = threadIdx.x; k < kRadixPasses * kRadixBins; k += 256) h[k] = 0;
    if (threadIdx.x < 64) {
        float lo[3], side;
        uint32_t bad;
        cube_from_partials(cube_part, cube_parts, lo, side, bad);
        const float scale = 2097152.0f / side;  // correctly rounded division
        if (threadIdx.x == 0) {
            s_cube[0] = lo[0];
            s_cube[1] = lo[1];
            s_cube[2] = lo[2];
            s_cube[3] = scale;
            if (blockIdx.x == 0) {
                for (int a = 0; a < 3; a++) prm->lo[a] = lo[a];
                prm->side = side;
                prm->scale = scale;
                prm->bad_input = bad;
                prm->n_nodes = 0;
                for (int q = 0; q < kRadixPasses; q++) prm->sort_ticket[q] = 0;
                prm->n_cut = 0;
                prm->n_top = 0;
            }
        }
    }
    __syncthreads();
    const float lx = s_cube[0], ly = s_cube[1], lz = s_cube[2], sc = s_cube[3];
    const uint32_t stride = gridDim.x * 256u;
    auto one = [&](uint32_t i, float x, float y, float z, float m) {
        const uint64_t key = (spread3(quantise(x, lx, sc)) << 2) | (spread3(quantise(y, ly, sc)) << 1) |
                             spread3(quantise(z, lz, sc));
        keys[i] = key;
        idx[i] = i;
        xs0[i] = make_float4(x, y, z, m);
        for (int p = 0; p < kRadixPasses; p++)
            atomicAdd(&h[p * kRadixBins + ((uint32_t)(key >> (p * kRadixBits)) & (kRadixBins - 1))], 1u);
    };
    uint32_t i = blockIdx.x * 256u + threadIdx.x;
    for (; i + 3u * stride < n; i += 4u * stride) {  // four particles' loads in flight
        float x[4], y[4], z[4], m[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint64_t j = i + (uint64_t)k * stride;
            x[k] = pos[3 * j];
            y[k] = pos[3 * j + 1];
            z[k] = pos[3 * j + 2];
            m[k] = mass[j];
        }
#pragma unroll
        for (int k = 0; k < 4; k++) one(i + k * stride, x[k], y[k], z[k], m[k]);
    }
    for (; i < n; i += stride) one(i, pos[3ull * i], pos[3ull * i + 1], pos[3ull * i + 2], mass[i]);
    __syncthreads();
    for (int k = threadIdx.x; k < kRadixPasses * kRadixBins; k += 256)
        part[(uint64_t)blockIdx.x * kRadixPasses * kRadixBins + k] = h[k];
    for (uint64_t w = (uint64_t)blockIdx.x * 256u + threadIdx.x; w < n_lb_words; w += stride) lb_words[w] = 0ull;
}

// Block p (1024 threads): first output slot of each digit in pass p. Thread
// (q, d) sums the digit-d counts of every fourth histogram block from q; the
// four partial sums are added, then scanned over digits.
__global__ __launch_bounds__(1024) void k_digit_offsets(const uint32_t *__restrict__ part, uint32_t nparts,
                                                        uint32_t *__restrict__ offs) {
    const int p = blockIdx.x, d = threadIdx.x & (kRadixBins - 1), q = threadIdx.x >> kRadixBits;
    // All loads first (nparts <= kSortHistBlocks), then the sum in block order.
    constexpr int kPer = kSortHistBlocks / 4;
    uint32_t c[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const uint32_t b = q + 4u * j;
        c[j] = b < nparts ? part[(uint64_t)b * kRadixPasses * kRadixBins + p * kRadixBins + d] : 0u;
    }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kPer; j++) s += c[j];
    __shared__ uint32_t sum[4][kRadixBins];
    __shared__ uint32_t wsum[4];
    sum[q][d] = s;
    __syncthreads();
    const int lane = d & 63, w = d >> 6;
    uint32_t v = 0, inc = 0;
    if (q == 0) {
        v = sum[0][d] + sum[1][d] + sum[2][d] + sum[3][d];
        inc = v;
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_up(inc, o, 64);
            if (lane >= o) inc += t;
        }
        if (lane == 63) wsum[w] = inc;
    }
    __syncthreads();  // every thread of the block reaches both barriers
    if (q == 0) {
        uint32_t off = 0;
        for (int k = 0; k < w; k++) off += wsum[k];
        offs[p * kRadixBins + d] = off + inc - v;
    }
}

// One pass over a tile of kTile keys. With W = kTileThreads / 64 waves, wave
// w owns elements [kTile t + w kTile/W, + kTile/W), lane l of round r element
// w kTile/W + 64 r + l, so (w, r, l) order is input order. The tile is reordered by digit in LDS and
// written out in that order, so consecutive threads store consecutive slots.
// kItems keys per thread: kTile = kTileThreads kItems.
template <int kItems, bool kGather>
__global__ __launch_bounds__(kTileThreads) void k_onesweep(const uint64_t *__restrict__ keys_in,
                                                  const uint32_t *__restrict__ vals_in, uint32_t n, int pass,
                                                  const uint32_t *__restrict__ digit_offs, uint64_t *lb_words,
                                                  DevParams *prm, uint64_t *__restrict__ keys_out,
                                                  uint32_t *__restrict__ vals_out, const float4 *__restrict__ xs0,
                                                  float4 *__restrict__ xs) {
    constexpr int kWaves = kTileThreads / 64, kTile = kTileThreads * kItems;
    static_assert(kWaves * kRadixBins * 4 <= kTile * 8, "counts fit in the key buffer");
    __shared__ uint64_t s_keys[kTile];  // first the per-wave digit counts, then the tile's keys by digit
    __shared__ uint32_t s_vals[kTile];
    __shared__ uint32_t s_delta[kRadixBins];  // output slot minus tile slot of each digit
    __shared__ uint32_t s_wsum[kRadixBins / 64];
    __shared__ uint32_t s_hist[kRadixBins];
    __shared__ uint32_t s_tile;
    uint32_t(*s_cnt)[kRadixBins] = reinterpret_cast<uint32_t(*)[kRadixBins]>(s_keys);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int shift = pass * kRadixBits;
    for (int k = threadIdx.x; k < kWaves * kRadixBins; k += kTileThreads) (&s_cnt[0][0])[k] = 0;
    if (threadIdx.x < kRadixBins) s_hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) s_tile = atomicAdd(&prm->sort_ticket[pass], 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t t0 = (uint64_t)tile * kTile;
    const uint32_t tile_n = (uint32_t)min<uint64_t>(kTile, n - t0);
    const uint64_t base = t0 + (uint64_t)w * (kTile / kWaves);

    uint64_t key[kItems];
    uint32_t val[kItems], rank[kItems];
    for (int r = 0; r < kItems; r++) {
        const uint64_t e = base + (uint64_t)r * 64 + lane;
        key[r] = e < n ? keys_in[e] : 0ull;
        val[r] = e < n ? vals_in[e] : 0u;
    }
    // The tile's digit counts first, published at once, so that later tiles
    // can add them while this one ranks its keys.
    for (int r = 0; r < kItems; r++)
        if (base + (uint64_t)r * 64 + lane < n) atomicAdd(&s_hist[(uint32_t)(key[r] >> shift) & (kRadixBins - 1)], 1u);
    __syncthreads();
    if (threadIdx.x < kRadixBins) lb_publish(lb_words + threadIdx.x, tile, kRadixBins, s_hist[threadIdx.x]);
    for (int r = 0; r < kItems; r++) {
        const bool valid = base + (uint64_t)r * 64 + lane < n;
        const uint32_t d = (uint32_t)(key[r] >> shift) & (kRadixBins - 1);
        uint64_t peers = __builtin_amdgcn_ballot_w64(valid);
        for (int b = 0; b < kRadixBits; b++) {
            const uint64_t m = __builtin_amdgcn_ballot_w64((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? m : ~m;
        }
        const uint32_t before = s_cnt[w][d];  // wave-private: no barrier, LDS is in order per wave
        rank[r] = before + __popcll(peers & lt_mask);
        if (valid && (peers & lt_mask) == 0ull) s_cnt[w][d] = before + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // Digit threads: tile totals, their scan over digits (the tile slot of
    // each digit's first element), the look-back over earlier tiles.
    uint32_t tot = 0, inc = 0;
    if (threadIdx.x < kRadixBins) {
        const int d = threadIdx.x;
        for (int k = 0; k < kWaves; k++) tot += s_cnt[k][d];
        inc = tot;
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_up(inc, o, 64);
            if (lane >= o) inc += t;
        }
        if (lane == 63) s_wsum[w] = inc;
    }
    __syncthreads();
    if (threadIdx.x < kRadixBins) {
        const int d = threadIdx.x;
        uint32_t local = inc - tot;
        for (int k = 0; k < w; k++) local += s_wsum[k];
        const uint32_t excl = lb_resolve(lb_words + d, tile, kRadixBins, tot, &prm->bad_input);
        s_delta[d] = digit_offs[pass * kRadixBins + d] + excl - local;
        uint32_t run = local;
        for (int k = 0; k < kWaves; k++) {  // in place: column d is this thread's alone
            const uint32_t c = s_cnt[k][d];
            s_cnt[k][d] = run;
            run += c;
        }
    }
    __syncthreads();
    uint32_t slot[kItems];
    for (int r = 0; r < kItems; r++) {
        const uint32_t d = (uint32_t)(key[r] >> shift) & (kRadixBins - 1);
        slot[r] = s_cnt[w][d] + rank[r];
    }
    __syncthreads();
    for (int r = 0; r < kItems; r++) {
        if (base + (uint64_t)r * 64 + lane < n) {
            s_keys[slot[r]] = key[r];
            s_vals[slot[r]] = val[r];
        }
    }
    __syncthreads();
    for (uint32_t j = threadIdx.x; j < tile_n; j += kTileThreads) {
        const uint64_t k = s_keys[j];
        const uint32_t v = s_vals[j];
        const uint32_t o = s_delta[(uint32_t)(k >> shift) & (kRadixBins - 1)] + j;
        keys_out[o] = k;
        vals_out[o] = v;
        if (kGather) xs[o] = xs0[v];
    }
}

}  // namespace

uint32_t morton_hist_blocks(int64_t n) { return (uint32_t)std::min<int64_t>(kSortHistBlocks, ceil_div(n, 256)); }

hipError_t launch_keys_and_sort(const float *pos, const float *mass, const Workspace &ws, hipStream_t s,
                                hipEvent_t after_keys) {
    const uint32_t n = (uint32_t)ws.n;
    const uint32_t nt = (uint32_t)ws.n_tiles;  // tiles of sort_tile_keys(n) keys
    const uint32_t hb = morton_hist_blocks(ws.n);
    const int cube_parts = (int)std::min<int64_t>(kCubeBlocks, ceil_div(ws.n, 256));  // as launch_cube
    // msum (at least n float4) holds the particles in input order until the
    // moments need it: the last pass gathers one aligned float4 per particle.
    k_morton_hist<<<hb, 256, 0, s>>>(pos, mass, ws.msum, n, ws.cube_part, cube_parts, ws.prm, ws.keys[0], ws.vals[0],
                                     ws.hist_part, ws.lb_words, (uint64_t)ws.n_lb_words);
    k_digit_offsets<<<kRadixPasses, 1024, 0, s>>>(ws.hist_part, hb, ws.digit_offs);
    if (after_keys) {
        hipError_t e = hipEventRecord(after_keys, s);
        if (e != hipSuccess) return e;
    }
    const int items = sort_tile_items(ws.n);
    for (int pass = 0; pass < kRadixPasses; pass++) {
        const int src = pass & 1, dst = src ^ 1;
        uint64_t *words = ws.lb_words + (uint64_t)pass * nt * kRadixBins;
        const bool last = pass + 1 == kRadixPasses;
#define ORR_ONESWEEP(ITEMS, GATHER)                                                                              \
    k_onesweep<ITEMS, GATHER><<<nt, kTileThreads, 0, s>>>(ws.keys[src], ws.vals[src], n, pass, ws.digit_offs, words, \
                                                          ws.prm, ws.keys[dst], ws.vals[dst],                      \
                                                          GATHER ? ws.msum : nullptr, GATHER ? ws.xs : nullptr)
        if (items == 2)
            last ? ORR_ONESWEEP(2, true) : ORR_ONESWEEP(2, false);
        else if (items == 4)
            last ? ORR_ONESWEEP(4, true) : ORR_ONESWEEP(4, false);
        else
            last ? ORR_ONESWEEP(8, true) : ORR_ONESWEEP(8, false);
#undef ORR_ONESWEEP
    }
    return hipGetLastError();
}

}  // namespace orr
