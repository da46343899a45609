// kda_mma.h -- matrix-core operand helpers shared by the prefill kernels.
//
// Ops<E> stages MFMA operands of element type E (bf16 or fp32).  `chain`
// accumulates A x B where B arrives as 16-row K blocks in accumulator layout
// (lane l: column l % 16, rows 4 (l / 16) + i) and A is read from row-major
// LDS in the matching K order; `gram` forms a 16 x 16 Gram over 128 channels.
#pragma once

#include "kda_device.h"

namespace kda {

// Operand helpers per staged element type.
template <typename E> struct Ops;

template <> struct Ops<__bf16> {
    typedef bf16x4 B4;  // one 16-row K block of a B operand, this lane's 4 elements
    static __device__ __forceinline__ B4 pack(f32x4 v) { return pack4(v); }
    static __device__ __forceinline__ f32x4 load4(const __bf16 *p) {
        bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
        f32x4 r = {(float)v.x, (float)v.y, (float)v.z, (float)v.w};
        return r;
    }
    static __device__ __forceinline__ bf16x4 load4raw(const __bf16 *p) {
        return *reinterpret_cast<const bf16x4 *>(p);
    }
    static __device__ __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d) {
        bf16x4 v;
        v.x = (__bf16)a; v.y = (__bf16)b; v.z = (__bf16)c; v.w = (__bf16)d;
        *reinterpret_cast<bf16x4 *>(p) = v;
    }
    // acc += sum_{kb < kb1} sum_i arow[16 kb + i] * B[kb][i], kb1 <= MAXKB; arow points
    // at A[row0 + lane%16][col0 + 4 (lane/16)].  kb1 folds to a constant once the
    // caller's loops are unrolled, so B stays in registers.
    template <int MAXKB>
    static __device__ __forceinline__ f32x4 chain(f32x4 acc, const __bf16 *arow, const B4 *B,
                                                  int kb1) {
#pragma unroll
        for (int kb = 0; kb < MAXKB; kb += 2) {
            if (kb + 1 < kb1) {
                bf16x4 a0 = *reinterpret_cast<const bf16x4 *>(arow + 16 * kb);
                bf16x4 a1 = *reinterpret_cast<const bf16x4 *>(arow + 16 * kb + 16);
                acc = mma_k32(join8(a0, a1), join8(B[kb], B[kb + 1]), acc);
            } else if (kb < kb1) {  // odd trailing block: same MFMA form as the pairs
                acc = mma_k16w(*reinterpret_cast<const bf16x4 *>(arow + 16 * kb), B[kb], acc);
            }
        }
        return acc;
    }
    // 16x16 Gram over 128 channels: lrow/rrow point at the rows of this lane's
    // A row / B column; f (nullable) scales the right operand per channel.
    static __device__ __forceinline__ f32x4 gram(const __bf16 *lrow, const __bf16 *rrow,
                                                 const float *f, int g4) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k0 = 32 * t + 8 * g4;
            bf16x8 a = join8(*reinterpret_cast<const bf16x4 *>(lrow + k0),
                             *reinterpret_cast<const bf16x4 *>(lrow + k0 + 4));
            bf16x4 b0 = *reinterpret_cast<const bf16x4 *>(rrow + k0);
            bf16x4 b1 = *reinterpret_cast<const bf16x4 *>(rrow + k0 + 4);
            if (f) {
                f32x4 f0 = *reinterpret_cast<const f32x4 *>(f + k0);
                f32x4 f1 = *reinterpret_cast<const f32x4 *>(f + k0 + 4);
                f32x4 x0 = {(float)b0.x, (float)b0.y, (float)b0.z, (float)b0.w};
                f32x4 x1 = {(float)b1.x, (float)b1.y, (float)b1.z, (float)b1.w};
                b0 = pack4(x0 * f0);
                b1 = pack4(x1 * f1);
            }
            acc = mma_k32(a, join8(b0, b1), acc);
        }
        return acc;
    }
};

template <> struct Ops<float> {
    typedef f32x4 B4;
    static __device__ __forceinline__ B4 pack(f32x4 v) { return v; }
    static __device__ __forceinline__ f32x4 load4(const float *p) {
        return *reinterpret_cast<const f32x4 *>(p);
    }
    static __device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
        f32x4 v = {a, b, c, d};
        *reinterpret_cast<f32x4 *>(p) = v;
    }
    template <int MAXKB>
    static __device__ __forceinline__ f32x4 chain(f32x4 acc, const float *arow, const B4 *B,
                                                  int kb1) {
#pragma unroll
        for (int kb = 0; kb < MAXKB; ++kb) {
            if (kb < kb1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mma_f32(arow[16 * kb + i], B[kb][i], acc);
            }
        }
        return acc;
    }
    static __device__ __forceinline__ f32x4 gram(const float *lrow, const float *rrow,
                                                 const float *f, int g4) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int k = 4 * t + g4;
            const float b = f ? rrow[k] * f[k] : rrow[k];
            acc = mma_f32(lrow[k], b, acc);
        }
        return acc;
    }
};

}  // namespace kda
