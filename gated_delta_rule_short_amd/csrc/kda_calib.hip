// kda_calib.hip -- streaming kernels of known byte counts (libkda_calib.so).
//
// Measurement only: they compute nothing of the mixer.  They give the HBM
// ceiling a memory-bound kernel can reach on this chip with a given access
// pattern, and kernels whose bytes are known exactly, against which the
// hardware byte counters are calibrated.
//   kda_calib_state_rmw: the state stream of one decode step -- one workgroup
//     of 512 threads per 64 KiB fp32 state, each thread reading 8 float4 of
//     whole 512-byte rows with non-temporal loads and writing them back in
//     place after one multiply, the same mapping as the decode kernel.
//   kda_calib_copy: dst = src, non-temporal, grid-stride, four float4 per lane
//     in flight (the fastest copy shape of a launch sweep on this chip).
//   kda_calib_fill: dst = value, non-temporal float4 stores, four per lane per
//     iteration, grid-stride.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_calib.h"

namespace {

typedef float f32x4c __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(512) state_rmw_kernel(float *state, float scale) {
    const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5;
    float *S = state + (size_t)blockIdx.x * 128 * 128;
    f32x4c st[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        st[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4c *>(S + (size_t)(rg + 16 * m) * 128 + 4 * cg));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        st[m] *= scale;
        __builtin_nontemporal_store(st[m], reinterpret_cast<f32x4c *>(S + (size_t)(rg + 16 * m) * 128 + 4 * cg));
    }
}

constexpr int kU = 4;  // float4 per lane per iteration

__global__ void __launch_bounds__(256) copy_kernel(const f32x4c *src, f32x4c *dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256 * kU;
    for (size_t base = (size_t)blockIdx.x * 256 * kU + threadIdx.x; base < n; base += stride) {
        f32x4c v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const size_t i = base + (size_t)u * 256;
            v[u] = i < n ? __builtin_nontemporal_load(src + i) : f32x4c{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const size_t i = base + (size_t)u * 256;
            if (i < n) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

__global__ void __launch_bounds__(256) fill_kernel(f32x4c *dst, size_t n, float value) {
    const size_t stride = (size_t)gridDim.x * 256 * kU;
    const f32x4c v = {value, value, value, value};
    for (size_t base = (size_t)blockIdx.x * 256 * kU + threadIdx.x; base < n; base += stride)
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const size_t i = base + (size_t)u * 256;
            if (i < n) __builtin_nontemporal_store(v, dst + i);
        }
}

unsigned grid_for(size_t n) {
    // 16384 workgroups of 256 lanes (64 per compute unit) at most, four float4 per lane
    const size_t want = (n + 256 * kU - 1) / (256 * kU);
    return (unsigned)(want < 16384 ? (want ? want : 1) : 16384);
}

}  // namespace

extern "C" {

int kda_calib_state_rmw(void *state, int64_t num_states, float scale, hipStream_t stream) {
    if (!state || num_states < 1 || num_states > ((int64_t)1 << 31) - 1 || (uintptr_t)state % 16)
        return 1;
    hipLaunchKernelGGL(state_rmw_kernel, dim3((unsigned)num_states), dim3(512), 0, stream,
                       static_cast<float *>(state), scale);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int kda_calib_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
    if (!dst || !src || bytes % 16 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return 1;
    const size_t n = bytes / 16;
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<const f32x4c *>(src), static_cast<f32x4c *>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int kda_calib_fill(void *dst, size_t bytes, float value, hipStream_t stream) {
    if (!dst || bytes % 16 || (uintptr_t)dst % 16) return 1;
    const size_t n = bytes / 16;
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n)), dim3(256), 0, stream, static_cast<f32x4c *>(dst), n,
                       value);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
