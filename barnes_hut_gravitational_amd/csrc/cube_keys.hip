// Root cube of the Morton keys.
//
// The orrery performance page ("Where one evaluation goes") puts a Morton
// sort in front of the tree build; the root cube is the reading stated in
// include/orr.h: corner = component-wise minimum, side = largest extent.
// HBM-bound streaming reduction (12 B of position + 4 B of mass per
// particle) into per-block partials; every block of the key kernel
// (sort.hip) combines them into the cube itself.
#include "orr_internal.h"

namespace orr {

namespace {

__device__ __forceinline__ float wave_min(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Per-block minimum and maximum of each axis plus an invalid-input flag.
// part[b] = (min x, min y, min z, max x, max y, max z, flag bits, unused).
__global__ __launch_bounds__(256) void k_cube_partial(const float *__restrict__ pos,
                                                      const float *__restrict__ mass, uint32_t n,
                                                      float *__restrict__ part) {
    float mn0 = INFINITY, mn1 = INFINITY, mn2 = INFINITY;
    float mx0 = -INFINITY, mx1 = -INFINITY, mx2 = -INFINITY;
    uint32_t bad = 0;
    const uint32_t stride = gridDim.x * 256u;
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
        for (int k = 0; k < 4; k++) {
            bad |= !(isfinite(x[k]) && isfinite(y[k]) && isfinite(z[k]) && isfinite(m[k]) && m[k] >= 0.0f);
            mn0 = fminf(mn0, x[k]);
            mn1 = fminf(mn1, y[k]);
            mn2 = fminf(mn2, z[k]);
            mx0 = fmaxf(mx0, x[k]);
            mx1 = fmaxf(mx1, y[k]);
            mx2 = fmaxf(mx2, z[k]);
        }
    }
    for (; i < n; i += stride) {
        float x = pos[3ull * i], y = pos[3ull * i + 1], z = pos[3ull * i + 2], m = mass[i];
        bad |= !(isfinite(x) && isfinite(y) && isfinite(z) && isfinite(m) && m >= 0.0f);
        mn0 = fminf(mn0, x);
        mn1 = fminf(mn1, y);
        mn2 = fminf(mn2, z);
        mx0 = fmaxf(mx0, x);
        mx1 = fmaxf(mx1, y);
        mx2 = fmaxf(mx2, z);
    }
    __shared__ float red[4][7];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float v[7] = {wave_min(mn0), wave_min(mn1), wave_min(mn2), wave_max(mx0), wave_max(mx1), wave_max(mx2),
                  __uint_as_float(__ballot(bad) != 0ull ? 1u : 0u)};
    if (lane == 0)
        for (int k = 0; k < 7; k++) red[w][k] = v[k];
    __syncthreads();
    if (threadIdx.x == 0) {
        float r[7];
        for (int k = 0; k < 7; k++) r[k] = red[0][k];
        for (int ww = 1; ww < 4; ww++) {
            for (int k = 0; k < 3; k++) r[k] = fminf(r[k], red[ww][k]);
            for (int k = 3; k < 6; k++) r[k] = fmaxf(r[k], red[ww][k]);
            r[6] = __uint_as_float(__float_as_uint(r[6]) | __float_as_uint(red[ww][6]));
        }
        for (int k = 0; k < 7; k++) part[8 * blockIdx.x + k] = r[k];
        part[8 * blockIdx.x + 7] = 0.0f;
    }
}

}  // namespace

hipError_t launch_cube(const float *pos, const float *mass, const Workspace &ws, hipStream_t s) {
    const uint32_t n = (uint32_t)ws.n;
    int blocks = (int)std::min<int64_t>(kCubeBlocks, ceil_div(ws.n, 256));
    k_cube_partial<<<blocks, 256, 0, s>>>(pos, mass, n, ws.cube_part);
    return hipGetLastError();
}

}  // namespace orr
