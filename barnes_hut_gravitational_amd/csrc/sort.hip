// Device-wide exclusive scan and the stable LSD radix sort of (key, index).
//
// The orrery performance page ("Where one evaluation goes", "The largest
// row") measures the host Morton sort as the largest single cost of an
// evaluation and names a device radix sort as the first thing to do; here it
// runs on the GPU. Equal keys keep ascending original index because every
// pass is stable and the payload starts as the identity.
//
// Each of the 8 passes (8-bit digits) is: tile histogram -> device-wide scan
// of the digit-major histogram -> stable scatter. Tiles are 256 threads x 16
// keys; within a tile, ranks are computed in 16 rounds of 256 keys, each wave
// finding its lanes' equal-digit peers with 8 ballots.
#include "orr_internal.h"

namespace orr {

namespace {

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Block-wide exclusive scan of one value per thread (256 threads); returns
// the exclusive prefix and writes the block total to *total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *total) {
    __shared__ uint32_t wsum[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc = wave_incl_scan(v, lane);
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (int k = 0; k < 4; k++) {
        if (k < w) off += wsum[k];
        tot += wsum[k];
    }
    __syncthreads();
    *total = tot;
    return off + inc - v;
}

__global__ __launch_bounds__(256) void k_scan_reduce(const uint32_t *__restrict__ in, uint64_t len,
                                                     uint32_t *__restrict__ part) {
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
    uint32_t s = 0;
    for (int r = 0; r < kTileItems; r++) {
        uint64_t e = base + (uint64_t)r * kTileThreads + threadIdx.x;
        if (e < len) s += in[e];
    }
    uint32_t tot;
    block_excl_scan(s, &tot);
    if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

// One block: exclusive scan of the tile partials in place; total -> *total.
__global__ __launch_bounds__(256) void k_scan_partials(uint32_t *__restrict__ part, uint32_t nparts,
                                                       uint32_t *__restrict__ total) {
    uint32_t carry = 0;
    for (uint32_t b0 = 0; b0 < nparts; b0 += 256) {
        uint32_t i = b0 + threadIdx.x;
        uint32_t v = i < nparts ? part[i] : 0u;
        uint32_t tot;
        uint32_t ex = block_excl_scan(v, &tot);
        if (i < nparts) part[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0 && total) *total = carry;
}

// Each thread owns 16 consecutive items of the tile.
__global__ __launch_bounds__(256) void k_scan_down(const uint32_t *in, uint32_t *out, uint64_t len,
                                                   const uint32_t *__restrict__ part) {
    const uint64_t base = (uint64_t)blockIdx.x * kTile + (uint64_t)threadIdx.x * kTileItems;
    uint32_t v[kTileItems];
    uint32_t s = 0;
    for (int k = 0; k < kTileItems; k++) {
        v[k] = (base + k < len) ? in[base + k] : 0u;
        s += v[k];
    }
    uint32_t tot;
    uint32_t run = part[blockIdx.x] + block_excl_scan(s, &tot);
    for (int k = 0; k < kTileItems; k++) {
        if (base + k < len) out[base + k] = run;
        run += v[k];
    }
}

// Digit histogram of one tile, digit-major: hist[d * n_tiles + tile].
__global__ __launch_bounds__(256) void k_radix_hist(const uint64_t *__restrict__ keys, uint32_t n, int shift,
                                                    uint32_t *__restrict__ hist, uint32_t n_tiles) {
    __shared__ uint32_t h[4][kRadixBins];
    const int w = threadIdx.x >> 6;
    for (int k = threadIdx.x; k < 4 * kRadixBins; k += 256) (&h[0][0])[k] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
    for (int r = 0; r < kTileItems; r++) {
        uint64_t e = base + (uint64_t)r * kTileThreads + threadIdx.x;
        if (e < n) atomicAdd(&h[w][(uint32_t)(keys[e] >> shift) & (kRadixBins - 1)], 1u);
    }
    __syncthreads();
    const int d = threadIdx.x;
    hist[(uint64_t)d * n_tiles + blockIdx.x] = h[0][d] + h[1][d] + h[2][d] + h[3][d];
}

// Stable scatter of one tile. offs[d * n_tiles + tile] = first output slot of
// this tile's keys with digit d (the scanned histogram).
__global__ __launch_bounds__(256) void k_radix_scatter(const uint64_t *__restrict__ keys_in,
                                                       const uint32_t *__restrict__ vals_in, uint32_t n,
                                                       int shift, const uint32_t *__restrict__ offs,
                                                       uint32_t n_tiles, uint64_t *__restrict__ keys_out,
                                                       uint32_t *__restrict__ vals_out) {
    __shared__ uint32_t s_base[kRadixBins];
    __shared__ uint32_t s_wc[4][kRadixBins];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    s_base[threadIdx.x] = offs[(uint64_t)threadIdx.x * n_tiles + blockIdx.x];
    for (int k = threadIdx.x; k < 4 * kRadixBins; k += 256) (&s_wc[0][0])[k] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
    for (int r = 0; r < kTileItems; r++) {
        const uint64_t e = base + (uint64_t)r * kTileThreads + threadIdx.x;
        const bool valid = e < n;
        uint64_t key = valid ? keys_in[e] : 0ull;
        uint32_t val = valid ? vals_in[e] : 0u;
        uint32_t d = (uint32_t)(key >> shift) & (kRadixBins - 1);
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < kRadixBits; b++) {
            bool bit = (d >> b) & 1u;
            uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t rank = __popcll(peers & lt_mask);
        const bool leader = valid && ((peers & lt_mask) == 0ull);
        if (leader) s_wc[w][d] = __popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pos = s_base[d] + rank;
            for (int k = 0; k < w; k++) pos += s_wc[k][d];
            keys_out[pos] = key;
            vals_out[pos] = val;
        }
        __syncthreads();
        {
            const int dd = threadIdx.x;
            s_base[dd] += s_wc[0][dd] + s_wc[1][dd] + s_wc[2][dd] + s_wc[3][dd];
            s_wc[0][dd] = s_wc[1][dd] = s_wc[2][dd] = s_wc[3][dd] = 0;
        }
        __syncthreads();
    }
}

// Particles into tree order: xs[k] = (pos[perm[k]], mass[perm[k]]).
__global__ __launch_bounds__(256) void k_gather(const float *__restrict__ pos, const float *__restrict__ mass,
                                                const uint32_t *__restrict__ perm, uint32_t n,
                                                float4 *__restrict__ xs) {
    const uint32_t k = blockIdx.x * 256u + threadIdx.x;
    if (k >= n) return;
    const uint64_t j = perm[k];
    xs[k] = make_float4(pos[3 * j], pos[3 * j + 1], pos[3 * j + 2], mass[j]);
}

}  // namespace

hipError_t launch_gather(const float *pos, const float *mass, const Workspace &ws, hipStream_t s) {
    k_gather<<<(unsigned)ceil_div(ws.n, 256), 256, 0, s>>>(pos, mass, ws.vals[0], (uint32_t)ws.n, ws.xs);
    return hipGetLastError();
}

hipError_t launch_exclusive_scan(const uint32_t *in, uint32_t *out, int64_t len, uint32_t *part,
                                 uint32_t *total, hipStream_t s) {
    const uint32_t nt = (uint32_t)ceil_div(len, kTile);
    k_scan_reduce<<<nt, 256, 0, s>>>(in, (uint64_t)len, part);
    k_scan_partials<<<1, 256, 0, s>>>(part, nt, total);
    k_scan_down<<<nt, 256, 0, s>>>(in, out, (uint64_t)len, part);
    return hipGetLastError();
}

hipError_t launch_sort(const Workspace &ws, hipStream_t s) {
    const uint32_t n = (uint32_t)ws.n;
    const uint32_t nt = (uint32_t)ws.n_tiles;
    for (int pass = 0; pass < kRadixPasses; pass++) {
        const int src = pass & 1, dst = src ^ 1;
        const int shift = pass * kRadixBits;
        k_radix_hist<<<nt, 256, 0, s>>>(ws.keys[src], n, shift, ws.hist, nt);
        hipError_t e = launch_exclusive_scan(ws.hist, ws.hist, (int64_t)kRadixBins * nt, ws.scan_part, nullptr, s);
        if (e != hipSuccess) return e;
        k_radix_scatter<<<nt, 256, 0, s>>>(ws.keys[src], ws.vals[src], n, shift, ws.hist, nt, ws.keys[dst],
                                           ws.vals[dst]);
    }
    return hipGetLastError();
}

}  // namespace orr
