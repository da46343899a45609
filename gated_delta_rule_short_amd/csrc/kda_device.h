// kda_device.h -- device-side helpers shared by the KDA kernels (gfx950).
//
// Element types, bf16 <-> fp32 conversion (hardware round-to-nearest-even),
// 64-lane wave reductions and thin wrappers over the CDNA4 matrix-core
// instructions used by the chunked prefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Pairs of elements: loads/stores of two adjacent channels in one access.
template <typename T> struct Pair;
template <> struct Pair<float> {
    typedef f32x2 vec;
    static __device__ __forceinline__ void load(const float *p, float &a, float &b) {
        f32x2 v = *reinterpret_cast<const f32x2 *>(p);
        a = v.x;
        b = v.y;
    }
    static __device__ __forceinline__ void store(float *p, float a, float b) {
        f32x2 v;
        v.x = a;
        v.y = b;
        *reinterpret_cast<f32x2 *>(p) = v;
    }
};
template <> struct Pair<__bf16> {
    typedef bf16x2 vec;
    static __device__ __forceinline__ void load(const __bf16 *p, float &a, float &b) {
        bf16x2 v = *reinterpret_cast<const bf16x2 *>(p);
        a = (float)v.x;
        b = (float)v.y;
    }
    static __device__ __forceinline__ void store(__bf16 *p, float a, float b) {
        bf16x2 v;
        v.x = (__bf16)a;
        v.y = (__bf16)b;
        *reinterpret_cast<bf16x2 *>(p) = v;
    }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// Logistic function on the VALU (exp is the device library's).
__device__ __forceinline__ float sigmoidf_dev(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------- MFMA
// 16x16 output tiles.  For every variant the accumulator (C/D) layout is:
// lane l holds column (l % 16) and rows 4*(l / 16) + i, i = 0..3.  The A
// operand holds row (l % 16), the B operand column (l % 16); both place the
// K elements of lane group l / 16 in the same slots, so any permutation of K
// applied identically to A and B leaves the product unchanged.

// bf16, K = 32: 8 K-elements per lane.
__device__ __forceinline__ f32x4 mma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// bf16, K = 16: 4 K-elements per lane.
__device__ __forceinline__ f32x4 mma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// fp32, K = 4: one K-element per lane.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 pack4(f32x4 v) {
    bf16x4 r;
    r.x = (__bf16)v.x;
    r.y = (__bf16)v.y;
    r.z = (__bf16)v.z;
    r.w = (__bf16)v.w;
    return r;
}
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
    r[0] = (__bf16)lo.x; r[1] = (__bf16)lo.y; r[2] = (__bf16)lo.z; r[3] = (__bf16)lo.w;
    r[4] = (__bf16)hi.x; r[5] = (__bf16)hi.y; r[6] = (__bf16)hi.z; r[7] = (__bf16)hi.w;
    return r;
}
__device__ __forceinline__ bf16x8 join8(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Index of the sequence holding token t: the largest n with cu[n] <= t.
__device__ __forceinline__ int find_seq(const int32_t *cu, int num_seqs, int64_t t) {
    int lo = 0, hi = num_seqs;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Sequence bounds from cu_seqlens, or equal splits when it is absent.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int64_t total, int num_seqs, int n,
                                           int64_t &start, int64_t &len) {
    if (cu) {
        start = cu[n];
        len = (int64_t)cu[n + 1] - start;
    } else {
        int64_t per = total / num_seqs;
        start = per * n;
        len = per;
    }
}

}  // namespace kda
