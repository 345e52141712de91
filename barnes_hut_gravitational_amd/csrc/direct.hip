// All-pairs float32 direct sum with the walk's term: the direct solver the
// orrery performance page measures the tree against ("Against the two
// solvers it has to beat"), here an O(n^2) reference on the device.
//
// One thread per target, 256 targets per block. Sources pass through LDS in
// tiles of 256 (x, y, z, m), staged with coalesced loads, and every thread
// adds a tile's terms in source order, so each target's sum runs over
// j = 0..n-1 in index order (the oracle's order) with the operations of
// term.h. Every lane of every wave does useful work on every row, so the
// kernel shows the issue-bound rate of the term itself.
#include "orr_internal.h"
#include "term.h"

namespace orr {

namespace {

constexpr uint32_t kDirectBlock = 256;

template <int kInv>
__global__ __launch_bounds__(kDirectBlock) void k_direct(const float *__restrict__ pos,
                                                         const float *__restrict__ mass, uint32_t n, float eps2,
                                                         float *__restrict__ acc) {
    __shared__ float4 src[kDirectBlock];
    const uint32_t i = blockIdx.x * kDirectBlock + threadIdx.x;
    const bool valid = i < n;  // lanes past n compute on a dummy target and store nothing
    const float xi = valid ? pos[3ull * i] : 0.0f;
    const float yi = valid ? pos[3ull * i + 1] : 0.0f;
    const float zi = valid ? pos[3ull * i + 2] : 0.0f;
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    for (uint32_t j0 = 0; j0 < n; j0 += kDirectBlock) {
        const uint32_t j = j0 + threadIdx.x;
        __syncthreads();  // the previous tile is consumed
        if (j < n) src[threadIdx.x] = make_float4(pos[3ull * j], pos[3ull * j + 1], pos[3ull * j + 2], mass[j]);
        __syncthreads();
        const uint32_t cnt = min(n - j0, kDirectBlock);
        uint32_t k = 0;
        for (; k + 4u <= cnt; k += 4u) {
            const float4 p0 = src[k], p1 = src[k + 1], p2 = src[k + 2], p3 = src[k + 3];
            add_term<kInv>(p0.w, p0.x - xi, p0.y - yi, p0.z - zi, eps2, ax, ay, az);
            add_term<kInv>(p1.w, p1.x - xi, p1.y - yi, p1.z - zi, eps2, ax, ay, az);
            add_term<kInv>(p2.w, p2.x - xi, p2.y - yi, p2.z - zi, eps2, ax, ay, az);
            add_term<kInv>(p3.w, p3.x - xi, p3.y - yi, p3.z - zi, eps2, ax, ay, az);
        }
        for (; k < cnt; k++) {
            const float4 p = src[k];
            add_term<kInv>(p.w, p.x - xi, p.y - yi, p.z - zi, eps2, ax, ay, az);
        }
    }
    if (valid) {
        acc[3ull * i] = ax;
        acc[3ull * i + 1] = ay;
        acc[3ull * i + 2] = az;
    }
}

}  // namespace

hipError_t launch_direct(const float *pos, const float *mass, int64_t n, float eps2, float *acc, hipStream_t s) {
    const unsigned blocks = (unsigned)ceil_div(n, kDirectBlock);
    // every r2 >= eps2 >= 2^-96 (the entry's range check on eps) lies in the
    // short inverse square root's domain
    k_direct<kInvFast><<<blocks, kDirectBlock, 0, s>>>(pos, mass, (uint32_t)n, eps2, acc);
    return hipGetLastError();
}

}  // namespace orr
