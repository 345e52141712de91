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

// targets (may be null): thread t sums for caller index targets[t], t <
// n_out; an index outside [0, n) gets NaN and reads nothing. Without targets
// thread t sums for particle t, t < n_out = n.
template <int kInv>
__global__ __launch_bounds__(kDirectBlock) void k_direct(const float *__restrict__ pos,
                                                         const float *__restrict__ mass, uint32_t n, float eps2,
                                                         const int64_t *__restrict__ targets, uint32_t n_out,
                                                         float *__restrict__ acc) {
    __shared__ float4 src[kDirectBlock];
    const uint32_t t = blockIdx.x * kDirectBlock + threadIdx.x;
    const bool out_ok = t < n_out;  // lanes past n_out compute on a dummy target and store nothing
    const int64_t it = !out_ok ? -1 : (targets ? targets[t] : (int64_t)t);
    const bool valid = it >= 0 && it < (int64_t)n;
    const uint64_t i = valid ? (uint64_t)it : 0ull;
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
    if (out_ok) {
        const float nan = __builtin_nanf("");
        acc[3ull * t] = valid ? ax : nan;
        acc[3ull * t + 1] = valid ? ay : nan;
        acc[3ull * t + 2] = valid ? az : nan;
    }
}

// Neumaier's compensated sum (1974): s holds the running sum, c the
// accumulated low-order parts lost by each addition; the result is s + c.
struct Compensated {
    double s = 0.0, c = 0.0;
    __device__ __forceinline__ void add(double x) {
        const double t = s + x;
        c += fabs(s) >= fabs(x) ? (s - t) + x : (x - t) + s;
        s = t;
    }
    __device__ __forceinline__ double value() const { return s + c; }
};

// Float64 reference for targets[t], t < n_out: the softened sum over every
// other particle j != i in index order, each term m_j d / (r2 sqrt(r2)) with
// r2 = dx*dx + dy*dy + dz*dz + eps^2 in IEEE double operations, summed with
// compensation per component (the compensated double-precision reference
// of the performance page, "Accuracy"). An index outside [0, n) gets NaN.
__global__ __launch_bounds__(kDirectBlock) void k_direct_fp64(const float *__restrict__ pos,
                                                              const float *__restrict__ mass, uint32_t n, double eps2,
                                                              const int64_t *__restrict__ targets, uint32_t n_out,
                                                              double *__restrict__ acc) {
    __shared__ float4 src[kDirectBlock];
    const uint32_t t = blockIdx.x * kDirectBlock + threadIdx.x;
    const bool out_ok = t < n_out;
    const int64_t it = out_ok ? targets[t] : -1;
    const bool valid = it >= 0 && it < (int64_t)n;
    const uint32_t i = valid ? (uint32_t)it : 0u;
    const double xi = pos[3ull * i], yi = pos[3ull * i + 1], zi = pos[3ull * i + 2];
    Compensated ax, ay, az;
    for (uint32_t j0 = 0; j0 < n; j0 += kDirectBlock) {
        const uint32_t j = j0 + threadIdx.x;
        __syncthreads();  // the previous tile is consumed
        if (j < n) src[threadIdx.x] = make_float4(pos[3ull * j], pos[3ull * j + 1], pos[3ull * j + 2], mass[j]);
        __syncthreads();
        const uint32_t cnt = min(n - j0, kDirectBlock);
        for (uint32_t k = 0; k < cnt; k++) {
            if (j0 + k == i) continue;
            const float4 p = src[k];
            const double dx = (double)p.x - xi, dy = (double)p.y - yi, dz = (double)p.z - zi;
            const double r2 = dx * dx + dy * dy + dz * dz + eps2;
            const double f = (double)p.w / (r2 * sqrt(r2));
            ax.add(f * dx);
            ay.add(f * dy);
            az.add(f * dz);
        }
    }
    if (out_ok) {
        const double nan = __builtin_nan("");
        acc[3ull * t] = valid ? ax.value() : nan;
        acc[3ull * t + 1] = valid ? ay.value() : nan;
        acc[3ull * t + 2] = valid ? az.value() : nan;
    }
}

}  // namespace

hipError_t launch_direct_fp64(const float *pos, const float *mass, int64_t n, double eps, const int64_t *targets,
                              int64_t n_out, double *acc, hipStream_t s) {
    const unsigned blocks = (unsigned)ceil_div(n_out, kDirectBlock);
    k_direct_fp64<<<blocks, kDirectBlock, 0, s>>>(pos, mass, (uint32_t)n, eps * eps, targets, (uint32_t)n_out, acc);
    return hipGetLastError();
}

hipError_t launch_direct(const float *pos, const float *mass, int64_t n, float eps2, const int64_t *targets,
                         int64_t n_out, float *acc, hipStream_t s) {
    const unsigned blocks = (unsigned)ceil_div(n_out, kDirectBlock);
    // every r2 >= eps2 >= 2^-96 (the entry's range check on eps) lies in the
    // short inverse square root's domain
    k_direct<kInvFast><<<blocks, kDirectBlock, 0, s>>>(pos, mass, (uint32_t)n, eps2, targets, (uint32_t)n_out, acc);
    return hipGetLastError();
}

}  // namespace orr
