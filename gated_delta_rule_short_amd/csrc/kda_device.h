// kda_device.h -- device-side helpers shared by the KDA kernels (gfx950).
//
// Element types, bf16 <-> fp32 conversion (hardware round-to-nearest-even),
// 64-lane wave reductions and thin wrappers over the CDNA4 matrix-core
// instructions used by the chunked prefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Pointer type of the LDS operand of the LDS-DMA load builtin.
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier that orders LDS accesses only: outstanding global loads and
// stores (LDS DMA included) stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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

// Sum over the 64 lanes of a wave; every lane receives the same value.  DPP
// moves combine lanes inside each 16-lane row (xor 1, xor 2, half-row mirror,
// row mirror), then the four row sums are read out as scalars.  Every lane has a
// source lane in these patterns, so bound_ctrl changes no value; set, it lets the
// compiler fold each move into the add that consumes it.
#define KDA_DPP(x, ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (x)), (ctrl), 0xf, 0xf, true))
__device__ __forceinline__ float wave_sum(float x) {
    x += KDA_DPP(x, 0xb1);   // quad_perm [1,0,3,2]
    x += KDA_DPP(x, 0x4e);   // quad_perm [2,3,0,1]
    x += KDA_DPP(x, 0x141);  // row_half_mirror
    x += KDA_DPP(x, 0x140);  // row_mirror
    const int xi = __builtin_bit_cast(int, x);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48)));
}

// 2^x on the transcendental unit (v_exp_f32); results below 2^-126 flush to 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic function: 1 / (1 + e^-x) with the hardware exp and reciprocal (1 ulp each).
__device__ __forceinline__ float sigmoidf_dev(float x) {
    return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-1.4426950408889634f * x));
}

// Sums of 16 per-row partials over the 64 lanes of a wave.  p[r] holds this
// lane's partial for row r.  Two butterfly steps across lane halves (xor 32,
// then xor 16) halve the row set per lane while doubling the lanes summed; the
// remaining 16 lanes of each row block are combined with DPP.  On return, every
// lane of 16-lane block b holds in out[j] the full sum of row 4 b + j.
//
// The butterflies use the gfx950 lane-swap instructions, which exchange half
// of one register with half of another inside the VALU (no LDS round trip):
// permlane32_swap(a, b) leaves (a.lo, b.lo) in the first result and (a.hi,
// b.hi) in the second, so their sum is a + a^32 in the low 32 lanes and
// b + b^32 in the high ones; permlane16_swap does the same for the even and odd
// 16-lane rows.  The two operands are always distinct rows' partials (with one
// value in both, this compiler has been seen to fold the two results into one).
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                    false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                    false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ void rows16_sum(float p[16], float out[4], int lane) {
    (void)lane;
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = swap32_sum(p[j], p[j + 8]);  // rows j (low half), j + 8 (high half)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x = swap16_sum(p[j], p[j + 4]);  // rows j, j + 4 of the half in even and odd 16-lane rows
        x += KDA_DPP(x, 0xb1);   // quad_perm [1,0,3,2]
        x += KDA_DPP(x, 0x4e);   // quad_perm [2,3,0,1]
        x += KDA_DPP(x, 0x141);  // row_half_mirror
        x += KDA_DPP(x, 0x140);  // row_mirror
        out[j] = x;
    }
}

// Value of row r (0..15) from rows16_sum's layout, as a wave-uniform scalar.
__device__ __forceinline__ float row_value(const float v[4], int r) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[r & 3]), 16 * (r >> 2)));
}

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

// Two paired conversions (v_cvt_pk_bf16_f32), joined as 32-bit words: with a
// four-wide conversion this compiler converts element by element and permutes
// when the result feeds an MFMA operand as well as a store.
__device__ __forceinline__ bf16x4 pack4(f32x4 v) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t lo = __builtin_convertvector((f32x2_t){v.x, v.y}, bf16x2_t);
    const bf16x2_t hi = __builtin_convertvector((f32x2_t){v.z, v.w}, bf16x2_t);
    const u32x2_t u = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    return __builtin_bit_cast(bf16x4, u);
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

// bf16, K = 16 issued as a K = 32 product whose upper K half is zero.  On gfx950
// an accumulator must not pass between the 16x16x32 and 16x16x16 forms without
// at least five wait states (measured; the compiler inserts none for that pair),
// so every accumulation chain that also holds K = 32 steps uses this form for its
// K = 16 steps.  The plain 16x16x16 form stays where the accumulator starts from
// zero or a vector result and ends in vector reads.
__device__ __forceinline__ f32x4 mma_k16w(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {};
    return mma_k32(join8(a, z), join8(b, z), c);
}

// Pool row of sequence n: slots[n] when a slot map is given, else n.  A slot
// outside [0, num_slots) gives -1, and the caller then skips the sequence.
__device__ __forceinline__ int pool_slot(const int32_t *slots, int num_slots, int n) {
    if (!slots) return n;
    const int s = slots[n];
    return (s >= 0 && s < num_slots) ? s : -1;
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
