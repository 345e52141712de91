// Morton keys with their digit histograms, and the stable sort of
// (key, index) into tree order with the gather of the particles.
//
// The orrery performance page ("Where one evaluation goes", "The largest
// row") measures the host Morton sort as the largest single cost of an
// evaluation and names a device radix sort as the first thing to do; here it
// runs on the GPU. The result is the stable sort by key: equal keys keep
// ascending original index.
//
// Structure. A 63-bit key splits into its high 32 bits H (bits 31..62) and
// its low 31 bits. Sorting by H alone takes 4 one-sweep LSD passes of 8-bit
// digits instead of 8; what remains is to order each run of equal H by the
// low bits, and in Morton order such runs are short: H holds the first 10
// levels of the key and the x and y bits of the 11th, so a run lies in one
// box of 2^-11 of the root side in x and y and 2^-10 in z, and on the
// Plummer, uniform and merger inputs runs average 1.0 to 1.5 keys and never
// exceed 30.
//   * k_morton_hist computes every key once and the 4 digit histograms of H;
//     k_digit_offsets turns them into the first output slot of each digit.
//   * k_onesweep, one launch per pass: a tile of 512 threads x 2, 4 or 8 keys
//     (by the input's size, sort_tile_items) takes a ticket (its position in
//     the output), counts its digits and publishes the counts at once, ranks
//     its keys stably inside each wave (lanes with the same digit found with
//     8 ballots), and then adds the counts of the tiles before it by
//     decoupled look-back: walking back over predecessors' published words,
//     four per step, until one carries an inclusive prefix. Tickets are taken
//     in the order blocks start, so every predecessor is running or done and
//     publishes its counts without waiting on anyone; each wait is
//     nevertheless bounded and reports an error. The tile is then reordered
//     by digit in LDS and written out in that order.
//   * k_sort_fix finishes the runs and gathers the particles: each thread
//     takes one position, finds its run from a window of keys in LDS (64
//     positions either side) and, for a run of at most 64, places its own
//     element at the run's start plus its stable rank by the low bits. A run
//     of 65 to 4,096 is sorted by the work-group holding its first position
//     (a bitonic sort in LDS of (low bits, position), unique values). A
//     longer run - more than 4,096 particles in one such box - is
//     measured by a 512-way search for its end (H only grows along the
//     array) and listed.
//   * k_sort_fallback, always launched, returns at once unless some run was
//     listed. Its persistent blocks then sort the listed runs' elements
//     together, as one virtual array (the runs in position order), by
//     (rank of the run, low 31 bits): LSD passes of the same tiles, driven
//     by one ticket counter (a histogram phase, then the passes in order,
//     each phase waiting for the one before it with a bounded wait). Digits
//     that are the same for every element are skipped. With more than 64
//     such runs the virtual array is the whole H-sorted array and the key
//     the full key: equal keys have equal H, so they are in index order
//     there, and a stable sort of it by the full key is the sort by
//     (key, index).
#include "checked.h"
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

// Publishes a tile's value for one digit: inclusive for tile 0, else an
// aggregate that successors can add while the tile works on.
__device__ __forceinline__ void lb_publish(uint64_t *words, uint32_t tile, uint32_t stride, uint32_t mine) {
    lb_store(words + (uint64_t)tile * stride, (tile == 0 ? kStInclusive : kStAggregate) | mine);
}

// Exclusive prefix over earlier tiles of one value, after lb_publish: walks
// back over the predecessors' words, kWin at a time, adding aggregates until
// an inclusive value, then publishes its own inclusive value. Sets *err on a
// wait that never ends. A window of 4 suits tiles that start in dispatch
// order (their predecessors are mostly resolved); tiles released together
// find only aggregates and walk back far, and take a wider window.
template <int kWin>
__device__ __forceinline__ uint32_t lb_resolve(uint64_t *words, uint32_t tile, uint32_t stride, uint32_t mine,
                                               uint32_t *err) {
    if (tile == 0) return 0;
    uint32_t excl = 0, spins = 0;
    int64_t t = (int64_t)tile - 1;
    while (true) {
        uint64_t v[kWin];
#pragma unroll
        for (int k = 0; k < kWin; k++)
            v[k] = t - k >= 0 ? lb_load(words + (uint64_t)(t - k) * stride) : kStInclusive;
        int used = 0;
        bool done = false;
#pragma unroll
        for (int k = 0; k < kWin; k++) {
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

// Keys and the identity payload; each block's 4 digit histograms of the high
// bits to part[block][pass][digit]; zeroes the look-back words of the 4
// passes; copies every particle as one float4 (x, y, z, m) in input order to
// xs0, which the gather reads from (one aligned load per particle instead of
// a 12-byte and a 4-byte one). Each block first forms the root cube from the
// partials; block 0 also stores it in prm with the input flag and resets the
// build's device counters.
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
                prm->n_particles = n;
                prm->n_nodes = 0;
                for (int q = 0; q < kRadixPasses; q++) prm->sort_ticket[q] = 0;
                prm->n_cut = 0;
                prm->n_top = 0;
                prm->sort_fallback = 0;
                prm->n_long = 0;
                prm->fb_ticket = 0;
                prm->fb_hist_done = 0;
                prm->fb_plan = 0;
                for (int q = 0; q <= kFullPasses; q++) prm->fb_done[q] = 0;
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
        const uint32_t hi = (uint32_t)(key >> kSortLowBits);
        for (int p = 0; p < kRadixPasses; p++)
            atomicAdd(&h[p * kRadixBins + ((hi >> (p * kRadixBits)) & (kRadixBins - 1))], 1u);
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

// Plain arrays in and out (the high-bit passes, and the fallback's
// scratch).
struct ArrayIO {
    const uint64_t *ki;
    const uint32_t *vi;
    uint64_t *ko;
    uint32_t *vo;
    __device__ __forceinline__ void load(uint64_t e, uint64_t &k, uint32_t &v) const {
        k = ki[e];
        v = vi[e];
    }
    __device__ __forceinline__ void store(uint64_t o, uint64_t k, uint32_t v) const {
        ko[o] = k;
        vo[o] = v;
    }
    __device__ __forceinline__ bool gathers() const { return false; }
    __device__ __forceinline__ float4 fetch(uint32_t) const { return float4{}; }
    __device__ __forceinline__ void store_with(uint64_t o, uint64_t k, uint32_t v, float4) const { store(o, k, v); }
};

// One stable pass over one tile of kTile = kTileThreads kItems keys, by digit
// (key >> shift) & 255, reading through io.load and writing through
// io.store. The tile is `tile`, or, with a ticket counter, the next ticket.
// digit_base[d]: the first output slot of digit d over all tiles; words:
// this pass's look-back words, [tile][digit]. With W = kTileThreads / 64
// waves, wave w owns elements [kTile t + w kTile/W, + kTile/W), lane l of
// round r element w kTile/W + 64 r + l, so (w, r, l) order is input order.
// The tile is reordered by digit in LDS and written out in that order, so
// consecutive threads store consecutive slots. An IO that also gathers a
// particle per element (io.gathers()) has each thread fetch all of its
// particles before it stores any, so that the random reads overlap.
template <int kItems, int kLbWin, class IO>
__device__ __forceinline__ void sweep_tile(const IO &io, uint32_t n, int shift, const uint32_t *digit_base,
                                           uint64_t *words, uint32_t *ticket, uint32_t tile_arg, uint32_t *err) {
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
    for (int k = threadIdx.x; k < kWaves * kRadixBins; k += kTileThreads) (&s_cnt[0][0])[k] = 0;
    if (threadIdx.x < kRadixBins) s_hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) s_tile = ticket ? atomicAdd(ticket, 1u) : tile_arg;
    __syncthreads();
    const uint32_t tile = __builtin_amdgcn_readfirstlane(s_tile);
    const uint64_t t0 = (uint64_t)tile * kTile;
    const uint32_t tile_n = (uint32_t)min<uint64_t>(kTile, n - t0);
    const uint64_t base = t0 + (uint64_t)w * (kTile / kWaves);

    uint64_t key[kItems];
    uint32_t val[kItems], rank[kItems];
    for (int r = 0; r < kItems; r++) {
        const uint64_t e = base + (uint64_t)r * 64 + lane;
        key[r] = 0ull;
        val[r] = 0u;
        if (e < n) io.load(e, key[r], val[r]);
    }
    // The tile's digit counts first, published at once, so that later tiles
    // can add them while this one ranks its keys.
    for (int r = 0; r < kItems; r++)
        if (base + (uint64_t)r * 64 + lane < n) atomicAdd(&s_hist[(uint32_t)(key[r] >> shift) & (kRadixBins - 1)], 1u);
    __syncthreads();
    if (threadIdx.x < kRadixBins) lb_publish(words + threadIdx.x, tile, kRadixBins, s_hist[threadIdx.x]);
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
        const uint32_t excl = lb_resolve<kLbWin>(words + d, tile, kRadixBins, tot, err);
        s_delta[d] = digit_base[d] + excl - local;
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
    if (io.gathers()) {
        float4 g[kItems];
        for (int r = 0; r < kItems; r++) {
            const uint32_t j = threadIdx.x + r * kTileThreads;
            g[r] = j < tile_n ? io.fetch(s_vals[j]) : float4{};
        }
        for (int r = 0; r < kItems; r++) {
            const uint32_t j = threadIdx.x + r * kTileThreads;
            if (j < tile_n) {
                const uint64_t k = s_keys[j];
                const uint32_t o = s_delta[(uint32_t)(k >> shift) & (kRadixBins - 1)] + j;
                if (guarded_lt(o, n, err)) io.store_with(o, k, s_vals[j], g[r]);
            }
        }
        return;
    }
    for (uint32_t j = threadIdx.x; j < tile_n; j += kTileThreads) {
        const uint64_t k = s_keys[j];
        const uint32_t v = s_vals[j];
        const uint32_t o = s_delta[(uint32_t)(k >> shift) & (kRadixBins - 1)] + j;
        if (guarded_lt(o, n, err)) io.store(o, k, v);  // always, unless a look-back wait gave up (flagged)
    }
}

// One pass of the high-bit sort: digit `pass` of H, one tile per block.
template <int kItems>
__global__ __launch_bounds__(kTileThreads) void k_onesweep(const uint64_t *__restrict__ keys_in,
                                                           const uint32_t *__restrict__ vals_in, uint32_t n, int pass,
                                                           const uint32_t *__restrict__ digit_offs, uint64_t *lb_words,
                                                           DevParams *prm, uint64_t *__restrict__ keys_out,
                                                           uint32_t *__restrict__ vals_out) {
    const ArrayIO io{keys_in, vals_in, keys_out, vals_out};
    sweep_tile<kItems, 4>(io, n, kSortLowBits + pass * kRadixBits, digit_offs + pass * kRadixBins, lb_words,
                          &prm->sort_ticket[pass], 0u, &prm->bad_input);
}

// Finishes the runs of equal high bits and gathers the particles. Input: the
// H-sorted keys and values; output: the sorted keys, values and particles.
// Block b owns positions [b B, b B + B), B = kFixThreads, and holds the keys
// of [b B - 64, b B + B + 64) in LDS with one bit per position that starts a
// run (a position whose H differs from its predecessor's; also the window's
// first slot and every position outside [1, n)). A thread at window slot q
// looks for its run's start in q's bit word and the one before (at least the
// 64 slots up to q) and for the next run's start in q's word and the one
// after (at least 64 slots past q). Finding both, its run [s, e) is exact;
// missing either, the run is longer than 64. Runs of 65 to kFixMaxRun keys
// are sorted by the block holding their first position; a longer one is
// measured and listed (first position, end) for the fallback, up to
// kMaxLongRuns of them. Block 0 also clears the fallback's digit counts.
__global__ __launch_bounds__(kFixThreads) void k_sort_fix(const uint64_t *__restrict__ keys_in,
                                                          const uint32_t *__restrict__ vals_in, uint32_t n,
                                                          const float4 *__restrict__ xs0,
                                                          uint64_t *__restrict__ keys_out,
                                                          uint32_t *__restrict__ vals_out, float4 *__restrict__ xs,
                                                          DevParams *__restrict__ prm, uint32_t *__restrict__ fb_hist,
                                                          uint2 *__restrict__ long_runs) {
    constexpr int kWin = kFixThreads + 2 * kFixHalo;
    constexpr int kWords = kWin / 64;
    constexpr int kMaxLong = kFixThreads / (kFixHalo + 1) + 1;  // long runs starting in one block
    static_assert(kWin % 64 == 0 && kWin <= kFixMaxRun, "window layout");
    __shared__ uint64_t s_buf[kFixMaxRun];  // the window's keys, then one long run's (low bits, position)
    __shared__ uint64_t s_head[kWords];
    __shared__ uint32_t s_long[kMaxLong];
    __shared__ uint32_t s_nlong, s_end;
    const int t = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kFixThreads;
    const int64_t p = t0 + t;
    const bool mine = p < n;
    const uint32_t v = mine ? vals_in[p] : 0u;  // issued early: the gather waits on it
    if (t == 0) s_nlong = 0;
    if (blockIdx.x == 0)
        for (int k = t; k < kFbHistWords; k += kFixThreads) fb_hist[k] = 0;
    for (int q = t; q < kWin; q += kFixThreads) {
        const int64_t g = t0 - kFixHalo + q;
        s_buf[q] = g >= 0 && g < n ? keys_in[g] : 0ull;
    }
    __syncthreads();
    for (int q = t; q < kWin; q += kFixThreads) {  // whole waves: kWin - kFixThreads is a multiple of 64
        const int64_t g = t0 - kFixHalo + q;
        const bool head =
            q == 0 || g <= 0 || g >= n || (s_buf[q] >> kSortLowBits) != (s_buf[q - 1] >> kSortLowBits);
        const uint64_t m = __builtin_amdgcn_ballot_w64(head);
        if ((q & 63) == 0) s_head[q >> 6] = m;
    }
    __syncthreads();
    if (mine) {
        const int q = kFixHalo + t, k = q >> 6;
        const uint64_t le = (2ull << (q & 63)) - 1;  // bits 0 .. q & 63
        // Run start: the last start at or before q, in this word or the one before.
        int s = -1;
        if (const uint64_t m = s_head[k] & le) s = 64 * k + 63 - __clzll(m);
        else if (const uint64_t m = s_head[k - 1]) s = 64 * (k - 1) + 63 - __clzll(m);
        // Run end: the first start after q, in this word or the next.
        int e = -1;
        if (const uint64_t m = s_head[k] & ~le) e = 64 * k + __ffsll((long long)m) - 1;
        else if (const uint64_t m = s_head[k + 1]) e = 64 * (k + 1) + __ffsll((long long)m) - 1;
        if (s >= 0 && e >= 0 && e - s <= kFixHalo) {
            const uint64_t key = s_buf[q];
            uint32_t rank = 0;
            for (int i = s; i < e; i++) {
                const uint64_t o = s_buf[i];
                rank += (o < key) | ((o == key) & (i < q));
            }
            const int64_t out = t0 - kFixHalo + s + rank;
            if (checked_lt((uint64_t)out, n, &prm->bad_input)) {
                keys_out[out] = key;
                vals_out[out] = v;
                if (checked_lt(v, n, &prm->bad_input)) xs[out] = xs0[v];
            }
        } else if (s == q) {
            s_long[atomicAdd(&s_nlong, 1u)] = (uint32_t)p;
        }
    }
    __syncthreads();
    // Loop bounds around barriers are read from LDS with readfirstlane: the
    // same for every thread, and known to the compiler to be uniform, so the
    // loops stay uniform control flow.
    const uint32_t nlong = __builtin_amdgcn_readfirstlane(s_nlong);
    for (uint32_t r = 0; r < nlong; r++) {
        const uint32_t S = __builtin_amdgcn_readfirstlane(s_long[r]);
        const uint64_t hs = keys_in[S] >> kSortLowBits;
        if (t == 0) s_end = ~0u;
        __syncthreads();
        // The run's end: the first position in (S, S + kFixMaxRun] past the
        // array or with other high bits.
        uint32_t end = ~0u;
        for (uint32_t c = S + 1; end == ~0u && c <= S + kFixMaxRun; c += kFixThreads) {
            const uint32_t j = c + t;
            if (j <= S + kFixMaxRun && (j >= n || (keys_in[j] >> kSortLowBits) != hs)) atomicMin(&s_end, j);
            __syncthreads();
            end = __builtin_amdgcn_readfirstlane(s_end);
            __syncthreads();
        }
        if (end == ~0u) {
            // Longer than kFixMaxRun. H only grows along the array, so the end
            // is the first position with greater H: a 512-way search, each
            // round narrowing [lo, hi] (the end lies in it, H = hs below lo)
            // to one sample interval.
            uint32_t lo = S + kFixMaxRun + 1, hi = n;
            while (lo < hi) {
                const uint32_t step = (hi - lo + kFixThreads - 1) / kFixThreads;
                if (t == 0) s_end = ~0u;
                __syncthreads();
                const uint64_t j = (uint64_t)lo + (uint64_t)t * step;
                if (j < hi && (keys_in[j] >> kSortLowBits) != hs) atomicMin(&s_end, (uint32_t)j);
                __syncthreads();
                const uint32_t f = __builtin_amdgcn_readfirstlane(s_end);
                __syncthreads();  // s_end is reset in the next round
                if (f == ~0u) {
                    const uint32_t last = lo + step * min<uint32_t>(kFixThreads - 1, (hi - 1 - lo) / step);
                    lo = last + 1;
                } else {
                    lo = f - lo >= step ? f - step + 1 : lo;
                    hi = f;
                }
            }
            if (t == 0) {
                const uint32_t i = atomicAdd(&prm->n_long, 1u);
                if (i < kMaxLongRuns) long_runs[i] = make_uint2(S, lo);
                atomicOr(&prm->sort_fallback, 1u);
            }
            continue;
        }
        const uint32_t len = end - S;
        uint32_t np = 128;
        while (np < len) np <<= 1;
        for (uint32_t i = t; i < np; i += kFixThreads)
            s_buf[i] = i < len ? ((keys_in[S + i] & 0x7fffffffull) << 12) | i : ~0ull;
        __syncthreads();
        for (uint32_t k = 2; k <= np; k <<= 1) {
            for (uint32_t j = k >> 1; j > 0; j >>= 1) {
                for (uint32_t i = t; i < np; i += kFixThreads) {
                    const uint32_t l = i ^ j;
                    if (l > i) {
                        const uint64_t a = s_buf[i], b = s_buf[l];
                        if ((a > b) == ((i & k) == 0)) {
                            s_buf[i] = b;
                            s_buf[l] = a;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (uint32_t i = t; i < len; i += kFixThreads) {
            const uint32_t src = S + (uint32_t)(s_buf[i] & 0xfffu);
            if (!checked_lt(src, n, &prm->bad_input)) continue;
            const uint32_t w = vals_in[src];
            keys_out[S + i] = keys_in[src];
            vals_out[S + i] = w;
            if (checked_lt(w, n, &prm->bad_input)) xs[S + i] = xs0[w];
        }
        __syncthreads();  // s_buf and s_end are reused by the next run
    }
}

// Bounded wait for a phase counter of the fallback to reach `target`.
__device__ __forceinline__ void wait_count(const uint32_t *c, uint32_t target, uint32_t *err) {
    uint32_t spins = 0;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++spins > kSpinLimit) {
            atomicOr(err, 2u);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// The fallback's virtual array: the listed runs in position order, run r at
// virtual positions [vb[r], vb[r + 1]), physical [s[r], s[r] + vb[r + 1] -
// vb[r]), all of whose keys have high bits h[r]. Its key is (r << 31) | low
// bits. In full mode it is the whole array with the full key (one "run").
struct RunTable {
    uint32_t s[kMaxLongRuns], vb[kMaxLongRuns + 1], h[kMaxLongRuns];
    uint32_t nr;
    uint32_t full;
};

// Reads the virtual array from the H-sorted input (src_a) or a plain
// scratch array; writes a plain scratch array or the output at the physical
// positions with the particles gathered (dst_out).
struct FallbackIO {
    const RunTable *tb;
    bool src_a, dst_out;
    const uint64_t *ki;
    const uint32_t *vi;
    uint64_t *ko;
    uint32_t *vo;
    const float4 *xs0;
    float4 *xs;
    uint32_t n;  // particles: gathered indices are checked against it
    uint32_t *err;  // the build's status word (checked build)
    __device__ __forceinline__ uint32_t run_of(uint64_t e) const {  // last r with vb[r] <= e
        uint32_t lo = 0, hi = tb->nr - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (tb->vb[mid] <= e) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    }
    __device__ __forceinline__ void load(uint64_t e, uint64_t &k, uint32_t &v) const {
        if (!src_a) {
            k = ki[e];
            v = vi[e];
        } else if (tb->full) {
            k = ki[e];
            v = vi[e];
        } else {
            const uint32_t r = run_of(e);
            const uint64_t ph = tb->s[r] + (e - tb->vb[r]);
            ORR_IF_CHECKED(if (!checked_lt(ph, n, err)) {
                k = 0ull;
                v = 0u;
                return;
            })
            k = ((uint64_t)r << kSortLowBits) | (ki[ph] & 0x7fffffffull);
            v = vi[ph];
        }
    }
    __device__ __forceinline__ void store(uint64_t o, uint64_t k, uint32_t v) const {
        if (!dst_out) {
            ko[o] = k;
            vo[o] = v;
            return;
        }
        uint64_t ph = o;
        if (!tb->full) {
            const uint32_t r = (uint32_t)(k >> kSortLowBits);
            ORR_IF_CHECKED(if (!checked_lt(r, tb->nr, err)) return;)
            ph = tb->s[r] + (o - tb->vb[r]);
            k = ((uint64_t)tb->h[r] << kSortLowBits) | (k & 0x7fffffffull);
        }
        ORR_IF_CHECKED(if (!checked_lt(ph, n, err)) return;)
        ko[ph] = k;
        vo[ph] = v;
        if (guarded_lt(v, n, err)) xs[ph] = xs0[v];
    }
    __device__ __forceinline__ bool gathers() const { return dst_out; }
    __device__ __forceinline__ float4 fetch(uint32_t v) const { return guarded_lt(v, n, err) ? xs0[v] : float4{}; }
    __device__ __forceinline__ void store_with(uint64_t o, uint64_t k, uint32_t v, float4 g) const {
        if (!dst_out) {
            ko[o] = k;
            vo[o] = v;
            return;
        }
        uint64_t ph = o;
        if (!tb->full) {
            const uint32_t r = (uint32_t)(k >> kSortLowBits);
            ORR_IF_CHECKED(if (!checked_lt(r, tb->nr, err)) return;)
            ph = tb->s[r] + (o - tb->vb[r]);
            k = ((uint64_t)tb->h[r] << kSortLowBits) | (k & 0x7fffffffull);
        }
        ORR_IF_CHECKED(if (!checked_lt(ph, n, err)) return;)
        ko[ph] = k;
        vo[ph] = v;
        xs[ph] = g;
    }
};

// The fallback, run only when k_sort_fix listed a run longer than
// kFixMaxRun (prm->sort_fallback). Work is handed out by one ticket counter:
// tickets [0, nt) are the histogram phase (the digit counts of each tile of
// the virtual array, and the tile's look-back words cleared), then nt
// tickets per pass slot. A block takes the next ticket only after finishing
// its current one, so the holders of all earlier tickets are running or
// done. The histogram tile that finishes last sets the plan (the digits that
// differ between keys) and then marks phase 0 done; a tile of slot j waits
// for the plan, skips when fewer than j digits differ, and otherwise waits
// until all nt tiles of slot j - 1 are done (release after a tile, acquire
// before one). Slot j sorts by the j-th differing digit, from the input
// (slot 1) or scratch x / y, to y / x or, for the last slot, the output;
// with no differing digit slot 1 copies the input to the output.
template <int kItems>
__global__ __launch_bounds__(kTileThreads) void k_sort_fallback(const uint64_t *keys_a, const uint32_t *vals_a,
                                                                uint64_t *keys_x, uint32_t *vals_x, uint64_t *keys_y,
                                                                uint32_t *vals_y, uint64_t *keys_out,
                                                                uint32_t *vals_out, uint32_t n, uint32_t *fb_hist,
                                                                const uint2 *long_runs, uint64_t *lb_words,
                                                                DevParams *prm, const float4 *__restrict__ xs0,
                                                                float4 *xs) {
    constexpr int kTile = kTileThreads * kItems;
    // Values that steer loops around barriers are read with readfirstlane:
    // prm is written by this kernel, so its loads are vector loads, which the
    // compiler cannot prove uniform.
    if (__builtin_amdgcn_readfirstlane(prm->sort_fallback) == 0) return;
    __shared__ RunTable tb;
    __shared__ uint32_t s_ticket, s_flag;
    __shared__ uint32_t s_base[kRadixBins];
    __shared__ uint32_t s_wsum[kRadixBins / 64];
    __shared__ uint32_t s_h[kFullPasses * kRadixBins];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // The run table: the listed runs ranked by first position.
    const uint32_t n_long = __builtin_amdgcn_readfirstlane(prm->n_long);
    const bool full = n_long > (uint32_t)kMaxLongRuns;
    if (threadIdx.x == 0) {
        tb.full = full;
        tb.nr = full ? 1u : n_long;
    }
    if (full) {
        if (threadIdx.x == 0) {
            tb.s[0] = 0;
            tb.vb[0] = 0;
            tb.vb[1] = n;
            tb.h[0] = 0;
        }
    } else if (threadIdx.x < n_long) {
        const uint2 me = long_runs[threadIdx.x];
        uint32_t rank = 0;
        for (uint32_t q = 0; q < n_long; q++) rank += long_runs[q].x < me.x;
        tb.s[rank] = me.x;
        tb.vb[rank + 1] = me.y - me.x;  // lengths for now
        tb.h[rank] = (uint32_t)(keys_a[me.x] >> kSortLowBits);
    }
    __syncthreads();
    if (!full && threadIdx.x == 0) {
        tb.vb[0] = 0;
        for (uint32_t r = 0; r < n_long; r++) tb.vb[r + 1] += tb.vb[r];
    }
    __syncthreads();
    const uint32_t m = __builtin_amdgcn_readfirstlane(tb.vb[tb.nr]);
    const int nd = __builtin_amdgcn_readfirstlane(full ? kFullPasses : kRunPasses);
    const uint32_t nt = __builtin_amdgcn_readfirstlane((m + kTile - 1) / kTile);
    const uint32_t total = __builtin_amdgcn_readfirstlane((1u + (uint32_t)nd) * nt);
    // Thread 0 takes the tickets; the loop is entered and left on the same
    // uniform value (readfirstlane after a barrier), and thread 0's work at
    // the end of an iteration is followed by a barrier, so every barrier in
    // the loop stays in uniform control flow.
    if (threadIdx.x == 0) s_ticket = atomicAdd(&prm->fb_ticket, 1u);
    __syncthreads();
    uint32_t ticket = __builtin_amdgcn_readfirstlane(s_ticket);
    while (ticket < total) {
        const uint32_t phase = ticket / nt, tile = ticket % nt;
        bool counted = false;  // phase 0 marks itself done through the plan
        if (phase == 0) {
            // Lanes with equal digits add their count once (clustered keys
            // share their high digits, and one LDS address per wave would
            // serialise 64 adds).
            for (int k = threadIdx.x; k < kFullPasses * kRadixBins; k += kTileThreads) s_h[k] = 0;
            __syncthreads();
            const FallbackIO io{&tb, true, false, keys_a, vals_a, nullptr, nullptr, nullptr, nullptr, n, &prm->bad_input};
            const uint64_t t0 = (uint64_t)tile * kTile;
            const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
            for (uint32_t r = 0; r < kItems; r++) {
                const uint64_t e = t0 + r * kTileThreads + threadIdx.x;
                const bool valid = e < m;
                uint64_t key = 0ull;
                uint32_t val = 0u;
                if (valid) io.load(e, key, val);
                const uint64_t live = __builtin_amdgcn_ballot_w64(valid);
                for (int q = 0; q < nd; q++) {
                    const uint32_t d = (uint32_t)(key >> (q * kRadixBits)) & (kRadixBins - 1);
                    uint64_t peers = live;
                    for (int b = 0; b < kRadixBits; b++) {
                        const uint64_t mk = __builtin_amdgcn_ballot_w64((d >> b) & 1u);
                        peers &= ((d >> b) & 1u) ? mk : ~mk;
                    }
                    if (valid && (peers & lt) == 0ull) atomicAdd(&s_h[q * kRadixBins + d], (uint32_t)__popcll(peers));
                }
            }
            __syncthreads();
            for (int k = threadIdx.x; k < nd * kRadixBins; k += kTileThreads)
                if (s_h[k]) atomicAdd(&fb_hist[k], s_h[k]);
            for (int k = threadIdx.x; k < nd * kRadixBins; k += kTileThreads) {
                const int q = k / kRadixBins, d = k % kRadixBins;
                lb_store(lb_words + ((uint64_t)q * nt + tile) * kRadixBins + d, 0ull);
            }
            // The last histogram tile sets the plan, then marks phase 0 done.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (threadIdx.x == 0) {
                const uint32_t prev =
                    __hip_atomic_fetch_add(&prm->fb_hist_done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                s_flag = prev + 1 == nt;
                if (s_flag) s_h[0] = 0;  // the plan's bits, gathered below
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(s_flag)) {
                uint32_t varies = 0;
                for (int k = threadIdx.x; k < nd * kRadixBins; k += kTileThreads) {
                    const uint32_t c =
                        __hip_atomic_load(&fb_hist[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (c != 0 && c != m) varies |= 1u << (k / kRadixBins);  // two or more digits occur
                }
                __syncthreads();  // s_h[0] is cleared before any thread adds to it
                if (varies) atomicOr(&s_h[0], varies);
                __syncthreads();
                if (threadIdx.x == 0) {
                    __hip_atomic_store(&prm->fb_plan, s_h[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_fetch_add(&prm->fb_done[0], nt, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            counted = true;
        } else {
            if (threadIdx.x == 0) {
                wait_count(&prm->fb_done[0], nt, &prm->bad_input);
                s_flag = __hip_atomic_load(&prm->fb_plan, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            const uint32_t plan = __builtin_amdgcn_readfirstlane(s_flag);
            const uint32_t slots = __popc(plan);
            const uint32_t slot = phase;  // 1-based
            if (slot <= max(slots, 1u)) {
                // Acquire by thread 0 after the previous slot, passed on to the
                // work-group by the barrier (its waves share one CU and its L1).
                if (threadIdx.x == 0) {
                    if (slot >= 2) wait_count(&prm->fb_done[slot - 1], nt, &prm->bad_input);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                }
                __syncthreads();
                const bool last = slot == max(slots, 1u);
                const uint64_t *ki = slot == 1 ? keys_a : (slot & 1) ? keys_y : keys_x;
                const uint32_t *vi = slot == 1 ? vals_a : (slot & 1) ? vals_y : vals_x;
                uint64_t *ko = last ? keys_out : (slot & 1) ? keys_x : keys_y;
                uint32_t *vo = last ? vals_out : (slot & 1) ? vals_x : vals_y;
                const FallbackIO io{&tb, slot == 1, last, ki, vi, ko, vo, xs0, xs, n, &prm->bad_input};
                if (slots == 0) {
                    // Every digit is the same: the input order is the sorted order.
                    const uint64_t t0 = (uint64_t)tile * kTile;
                    for (uint64_t e = t0 + threadIdx.x; e < m && e < t0 + kTile; e += kTileThreads) {
                        uint64_t k;
                        uint32_t v;
                        io.load(e, k, v);
                        io.store(e, k, v);
                    }
                } else {
                    uint32_t q = 0;  // the slot-th differing digit
                    for (uint32_t b = plan, j = 0; b; b &= b - 1)
                        if (++j == slot) q = __ffs(b) - 1;
                    // First output slot of each digit: the exclusive scan of the counts.
                    uint32_t c = 0, inc = 0;
                    if (threadIdx.x < kRadixBins) {
                        c = __hip_atomic_load(&fb_hist[q * kRadixBins + threadIdx.x], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                        inc = c;
                        for (int o = 1; o < 64; o <<= 1) {
                            const uint32_t u = __shfl_up(inc, o, 64);
                            if (lane >= o) inc += u;
                        }
                        if (lane == 63) s_wsum[w] = inc;
                    }
                    __syncthreads();
                    if (threadIdx.x < kRadixBins) {
                        uint32_t off = inc - c;
                        for (int k = 0; k < w; k++) off += s_wsum[k];
                        s_base[threadIdx.x] = off;
                    }
                    __syncthreads();
                    sweep_tile<kItems, 16>(io, m, (int)q * kRadixBits, s_base,
                                           lb_words + (uint64_t)(slot - 1) * nt * kRadixBins, nullptr, tile,
                                           &prm->bad_input);
                }
            }
        }
        // One release per tile, by thread 0: each wave first waits until its
        // own stores have reached the L2 (the barrier alone does not wait for
        // them), so thread 0's L2 write-back covers the whole tile.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            if (!counted)
                __hip_atomic_fetch_add(&prm->fb_done[phase], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            s_ticket = atomicAdd(&prm->fb_ticket, 1u);
        }
        __syncthreads();
        ticket = __builtin_amdgcn_readfirstlane(s_ticket);
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
    // moments need it: the gather reads one aligned float4 per particle.
    k_morton_hist<<<hb, 256, 0, s>>>(pos, mass, ws.msum, n, ws.cube_part, cube_parts, ws.prm, ws.keys[1], ws.vals[1],
                                     ws.hist_part, ws.lb_words, (uint64_t)kRadixPasses * nt * kRadixBins);
    k_digit_offsets<<<kRadixPasses, 1024, 0, s>>>(ws.hist_part, hb, ws.digit_offs);
    if (after_keys) {
        hipError_t e = hipEventRecord(after_keys, s);
        if (e != hipSuccess) return e;
    }
    const int items = sort_tile_items(ws.n);
    for (int pass = 0; pass < kRadixPasses; pass++) {  // keys[1] -> keys[0] -> ... -> keys[1]
        const int src = (pass & 1) ^ 1, dst = src ^ 1;
        uint64_t *words = ws.lb_words + (uint64_t)pass * nt * kRadixBins;
#define ORR_ONESWEEP(ITEMS)                                                                                      \
    k_onesweep<ITEMS><<<nt, kTileThreads, 0, s>>>(ws.keys[src], ws.vals[src], n, pass, ws.digit_offs, words, ws.prm, \
                                                  ws.keys[dst], ws.vals[dst])
        if (items == 2)
            ORR_ONESWEEP(2);
        else if (items == 4)
            ORR_ONESWEEP(4);
        else
            ORR_ONESWEEP(8);
#undef ORR_ONESWEEP
    }
    uint2 *long_runs = reinterpret_cast<uint2 *>(ws.hist_part + kFbHistWords);
    k_sort_fix<<<(uint32_t)ceil_div(ws.n, kFixThreads), kFixThreads, 0, s>>>(
        ws.keys[1], ws.vals[1], n, ws.msum, ws.keys[0], ws.vals[0], ws.xs, ws.prm, ws.hist_part, long_runs);
    // The fallback's ping-pong scratch: the node records, not written before
    // the build (32 bytes per node, at least n nodes): x at byte 0, y at 16 n,
    // 12 bytes per element each.
    uint64_t *keys_x = reinterpret_cast<uint64_t *>(ws.nodes);
    uint32_t *vals_x = reinterpret_cast<uint32_t *>(keys_x + ws.n);
    uint64_t *keys_y = keys_x + 2 * ws.n;
    uint32_t *vals_y = reinterpret_cast<uint32_t *>(keys_y + ws.n);
#define ORR_FALLBACK(ITEMS)                                                                                         \
    k_sort_fallback<ITEMS><<<kFallbackBlocks, kTileThreads, 0, s>>>(ws.keys[1], ws.vals[1], keys_x, vals_x, keys_y, \
                                                                    vals_y, ws.keys[0], ws.vals[0], n, ws.hist_part, \
                                                                    long_runs, ws.lb_words, ws.prm, ws.msum, ws.xs)
    if (items == 2)
        ORR_FALLBACK(2);
    else if (items == 4)
        ORR_FALLBACK(4);
    else
        ORR_FALLBACK(8);
#undef ORR_FALLBACK
    return hipGetLastError();
}

}  // namespace orr
