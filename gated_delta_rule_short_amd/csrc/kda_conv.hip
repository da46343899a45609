// kda_conv.hip -- causal depthwise convolution of width 4 over packed sequences,
// and the conv-state tail update shared with the prefill.
//
// Source: "GLM-5.3-Flash im Detail" (flozi.net), section "Sequenz-Mixing":
// q, k and v pass through a causal depthwise convolution of width four; the
// conv state is kept beside the recurrent state (same section, state size).
//
// Both kernels stream HBM once: each thread owns two adjacent channels and a run
// of tokens, keeping the three-token window in registers, so consecutive lanes
// read consecutive channels of one token (coalesced rows).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kConvThreads = 256;
constexpr int kConvTokens = 32;  // tokens per thread

template <typename T, bool SILU>
__global__ void __launch_bounds__(kConvThreads)
short_conv_kernel(const T *__restrict__ x, T *__restrict__ y, int64_t total, int C,
                  const float *__restrict__ w, const float *__restrict__ bias,
                  const T *__restrict__ cs_in, const int32_t *__restrict__ cu, int num_seqs) {
    const int c = 2 * (blockIdx.y * kConvThreads + threadIdx.x);
    if (c >= C) return;
    const int64_t t0 = (int64_t)blockIdx.x * kConvTokens;
    if (t0 >= total) return;
    const int64_t t1 = min(total, t0 + (int64_t)kConvTokens);
    const bool pair = (c + 1) < C;
    const bool vec_ok = (C & 1) == 0;  // rows start on a pair boundary

    float wa[4], wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        wa[j] = w[4 * c + j];
        wb[j] = pair ? w[4 * (c + 1) + j] : 0.f;
    }
    const float ba = bias ? bias[c] : 0.f;
    const float bb = (bias && pair) ? bias[c + 1] : 0.f;

    auto load2 = [&](const T *p, float &a, float &b) {
        if (pair && vec_ok) {
            Pair<T>::load(p, a, b);
        } else {
            a = to_f32(p[0]);
            b = pair ? to_f32(p[1]) : 0.f;
        }
    };

    const int64_t per = cu ? 0 : total / num_seqs;
    int n = cu ? find_seq(cu, num_seqs, t0) : (int)(t0 / per);
    int64_t s0, len;
    seq_bounds(cu, total, num_seqs, n, s0, len);

    // window[j] = x[t - 3 + j] for j = 0..2
    float ha[3], hb[3];
    auto fill_history = [&](int64_t t) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t p = t - 3 + j;
            if (p >= s0) {
                load2(x + p * C + c, ha[j], hb[j]);
            } else if (cs_in) {
                load2(cs_in + ((int64_t)n * 3 + (3 + (p - s0))) * C + c, ha[j], hb[j]);
            } else {
                ha[j] = 0.f;
                hb[j] = 0.f;
            }
        }
    };
    fill_history(t0);

    for (int64_t t = t0; t < t1; ++t) {
        if (t >= s0 + len) {  // next non-empty sequence starts at t
            while ((int64_t)s0 + len <= t) {
                ++n;
                seq_bounds(cu, total, num_seqs, n, s0, len);
            }
            fill_history(t);
        }
        float xa, xb;
        load2(x + t * C + c, xa, xb);
        float ya = ba + wa[0] * ha[0] + wa[1] * ha[1] + wa[2] * ha[2] + wa[3] * xa;
        float yb = bb + wb[0] * hb[0] + wb[1] * hb[1] + wb[2] * hb[2] + wb[3] * xb;
        if (SILU) {
            ya = ya * sigmoidf_dev(ya);
            yb = yb * sigmoidf_dev(yb);
        }
        if (pair && vec_ok) {
            Pair<T>::store(y + t * C + c, ya, yb);
        } else {
            y[t * C + c] = from_f32<T>(ya);
            if (pair) y[t * C + c + 1] = from_f32<T>(yb);
        }
        ha[0] = ha[1]; ha[1] = ha[2]; ha[2] = xa;
        hb[0] = hb[1]; hb[1] = hb[2]; hb[2] = xb;
    }
}

// Vector path: each thread owns 16 bytes of channels (8 bf16 or 4 fp32) and a
// run of kVecTokens tokens.  A run whose window (3 history rows + the run) lies
// inside one sequence loads all its rows up front with 16-byte non-temporal
// loads; runs that touch a sequence start or end take the per-token path.  32
// tokens per run re-read 3/32 of the rows for the history (16 re-read 3/16 and
// ran 13 % slower on 137,314 x 24,576 bf16; 48 measured the same as 32 with 64
// more VGPRs).
constexpr int kVecTokens = 32;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(u32x4 r, float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(r[i] << 16);
            v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ u32x4 pack(const float (&v)[8]) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x2 p2 = {(__bf16)v[2 * i], (__bf16)v[2 * i + 1]};
            r[i] = __builtin_bit_cast(uint32_t, p2);
        }
        return r;
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(u32x4 r, float (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
    }
    static __device__ __forceinline__ u32x4 pack(const float (&v)[4]) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(v[i]);
        return r;
    }
};

template <typename T, bool SILU>
__global__ void __launch_bounds__(kConvThreads)
short_conv_vec_kernel(const T *__restrict__ x, T *__restrict__ y, int64_t total, int C,
                      const float *__restrict__ w, const float *__restrict__ bias,
                      const T *__restrict__ cs_in, const int32_t *__restrict__ cu, int num_seqs) {
    typedef Vec16<T> V;
    constexpr int NV = V::N;
    // flat grid, channel blocks fastest: workgroups in flight together cover whole
    // rows.  The launcher picks the block width so that the block count per run is
    // a multiple of 8 where it can: workgroup b runs on XCD b mod 8, so every run of
    // a channel block then lands on the same XCD (and L2) as the run before it,
    // whose last rows are this run's history rows.
    const int bt = blockDim.x;
    const int nblk = (C / NV + bt - 1) / bt;
    const int64_t run = blockIdx.x / nblk;
    const int c = NV * ((int)(blockIdx.x - run * nblk) * bt + threadIdx.x);
    if (c >= C) return;
    const int64_t t0 = run * kVecTokens;
    const int64_t t1 = min(total, t0 + (int64_t)kVecTokens);
    float wt[NV][4], bs[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(w + 4 * (c + i));
#pragma unroll
        for (int j = 0; j < 4; ++j) wt[i][j] = a[j];
        bs[i] = bias ? bias[c + i] : 0.f;
    }
    auto emit = [&](int64_t t, const float (&h0)[NV], const float (&h1)[NV], const float (&h2)[NV],
                    const float (&cur)[NV]) {
        float o[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float a = fmaf(wt[i][0], h0[i], bs[i]);
            a = fmaf(wt[i][1], h1[i], a);
            a = fmaf(wt[i][2], h2[i], a);
            a = fmaf(wt[i][3], cur[i], a);
            if (SILU) a *= sigmoidf_dev(a);
            o[i] = a;
        }
        __builtin_nontemporal_store(V::pack(o), reinterpret_cast<u32x4 *>(y + t * C + c));
    };
    int n = cu ? find_seq(cu, num_seqs, t0) : (int)(t0 / (total / num_seqs));
    int64_t s0, len;
    seq_bounds(cu, total, num_seqs, n, s0, len);
    if (t0 - 3 >= s0 && t1 <= s0 + len && t1 - t0 == kVecTokens) {
        u32x4 raw[kVecTokens + 3];
#pragma unroll
        for (int r = 0; r < kVecTokens + 3; ++r)
            raw[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + (t0 - 3 + r) * C + c));
#pragma unroll
        for (int r = 0; r < kVecTokens; ++r) {
            float h0[NV], h1[NV], h2[NV], cur[NV];
            V::unpack(raw[r], h0);
            V::unpack(raw[r + 1], h1);
            V::unpack(raw[r + 2], h2);
            V::unpack(raw[r + 3], cur);
            emit(t0 + r, h0, h1, h2, cur);
        }
        return;
    }
    // per-token path: history from this sequence, its conv state, or zeros
    auto row = [&](int64_t p, float (&v)[NV]) {
        if (p >= s0) {
            V::unpack(*reinterpret_cast<const u32x4 *>(x + p * C + c), v);
        } else if (cs_in) {
            V::unpack(*reinterpret_cast<const u32x4 *>(cs_in + ((int64_t)n * 3 + (3 + (p - s0))) * C + c), v);
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) v[i] = 0.f;
        }
    };
    for (int64_t t = t0; t < t1; ++t) {
        while (t >= s0 + len) {  // next sequence (empty ones are skipped)
            ++n;
            seq_bounds(cu, total, num_seqs, n, s0, len);
        }
        float h0[NV], h1[NV], h2[NV], cur[NV];
        row(t - 3, h0);
        row(t - 2, h1);
        row(t - 1, h2);
        row(t, cur);
        emit(t, h0, h1, h2, cur);
    }
}

template <typename T>
__global__ void __launch_bounds__(kConvThreads)
conv_tail_kernel(const T *__restrict__ s0p, const T *__restrict__ s1p, const T *__restrict__ s2p,
                 int c0, int c1, int c2, int64_t total, const T *cs_in, T *cs_out,
                 const int32_t *__restrict__ cu, int num_seqs, const int32_t *slots,
                 int num_slots) {
    const int CC = c0 + c1 + c2;
    const int c = blockIdx.y * kConvThreads + threadIdx.x;
    const int n = blockIdx.x;
    const int slot = pool_slot(slots, num_slots, n);  // conv-state row of sequence n
    if (c >= CC || slot < 0) return;
    int64_t st, len;
    seq_bounds(cu, total, num_seqs, n, st, len);
    const T *src;
    int ch, cc;
    if (c < c0) { src = s0p; ch = c0; cc = c; }
    else if (c < c0 + c1) { src = s1p; ch = c1; cc = c - c0; }
    else { src = s2p; ch = c2; cc = c - c0 - c1; }
    T vals[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int64_t p = len - 3 + s;
        if (p >= 0) vals[s] = src[(st + p) * ch + cc];
        else if (cs_in) vals[s] = cs_in[((int64_t)slot * 3 + (3 + p)) * CC + c];
        else vals[s] = from_f32<T>(0.f);
    }
    // every thread reads its own (slot, c) entries before writing them: in place is safe
#pragma unroll
    for (int s = 0; s < 3; ++s) cs_out[((int64_t)slot * 3 + s) * CC + c] = vals[s];
}

template <typename T>
static hipError_t short_conv_t(const void *x, void *y, int64_t T_, int C, const float *w,
                               const float *b, const void *cs_in, const int32_t *cu, int N,
                               bool silu, hipStream_t s) {
    if (T_ == 0) return hipSuccess;
    constexpr int NV = Vec16<T>::N;
    int vt = kConvThreads;  // block width of the vector path (see short_conv_vec_kernel)
    for (const int cand : {256, 192, 128, 64})
        if (((C / NV + cand - 1) / cand) % 8 == 0) {
            vt = cand;
            break;
        }
    const int64_t nblk_v = (C / NV + vt - 1) / vt;
    const int64_t items_v = ((T_ + kVecTokens - 1) / kVecTokens) * nblk_v * vt;
    const bool vec = (C % NV) == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)y % 16) == 0 &&
                     (cs_in == nullptr || ((uintptr_t)cs_in % 16) == 0) && ((uintptr_t)w % 16) == 0 &&
                     items_v < (int64_t(1) << 32);  // one flat grid dimension
    if (vec) {
        dim3 grid((unsigned)(items_v / vt));
        if (silu)
            hipLaunchKernelGGL((short_conv_vec_kernel<T, true>), grid, dim3(vt), 0, s,
                               (const T *)x, (T *)y, T_, C, w, b, (const T *)cs_in, cu, N);
        else
            hipLaunchKernelGGL((short_conv_vec_kernel<T, false>), grid, dim3(vt), 0, s,
                               (const T *)x, (T *)y, T_, C, w, b, (const T *)cs_in, cu, N);
        trace("short_conv_vec_kernel<%s, silu=%d> grid=(%u) block=%d lds=0", sizeof(T) == 2 ? "bf16" : "f32",
              (int)silu, grid.x, vt);
        return hipGetLastError();
    }
    // tokens on x (up to 2^31 blocks), channel pairs on y
    dim3 grid((unsigned)((T_ + kConvTokens - 1) / kConvTokens),
              (unsigned)(((C + 1) / 2 + kConvThreads - 1) / kConvThreads));
    if (silu)
        hipLaunchKernelGGL((short_conv_kernel<T, true>), grid, dim3(kConvThreads), 0, s,
                           (const T *)x, (T *)y, T_, C, w, b, (const T *)cs_in, cu, N);
    else
        hipLaunchKernelGGL((short_conv_kernel<T, false>), grid, dim3(kConvThreads), 0, s,
                           (const T *)x, (T *)y, T_, C, w, b, (const T *)cs_in, cu, N);
    trace("short_conv_kernel<%s, silu=%d> grid=(%u,%u) block=%d lds=0", sizeof(T) == 2 ? "bf16" : "f32",
          (int)silu, grid.x, grid.y, kConvThreads);
    return hipGetLastError();
}

hipError_t launch_short_conv(kda_dtype dt, const void *x, void *y, int64_t T_, int C,
                             const float *w, const float *b, const void *cs_in,
                             const int32_t *cu, int N, bool silu, hipStream_t s) {
    if (dt == KDA_BF16) return short_conv_t<__bf16>(x, y, T_, C, w, b, cs_in, cu, N, silu, s);
    return short_conv_t<float>(x, y, T_, C, w, b, cs_in, cu, N, silu, s);
}

hipError_t launch_conv_tail(kda_dtype dt, const void *const src[3], const int ch[3], int64_t T_,
                            const void *cs_in, void *cs_out, const int32_t *cu, int N,
                            const int32_t *slots, int num_slots, hipStream_t s) {
    const int CC = ch[0] + ch[1] + ch[2];
    dim3 grid((unsigned)N, (unsigned)((CC + kConvThreads - 1) / kConvThreads));
    if (dt == KDA_BF16)
        hipLaunchKernelGGL((conv_tail_kernel<__bf16>), grid, dim3(kConvThreads), 0, s,
                           (const __bf16 *)src[0], (const __bf16 *)src[1], (const __bf16 *)src[2],
                           ch[0], ch[1], ch[2], T_, (const __bf16 *)cs_in, (__bf16 *)cs_out, cu, N,
                           slots, num_slots);
    else
        hipLaunchKernelGGL((conv_tail_kernel<float>), grid, dim3(kConvThreads), 0, s,
                           (const float *)src[0], (const float *)src[1], (const float *)src[2],
                           ch[0], ch[1], ch[2], T_, (const float *)cs_in, (float *)cs_out, cu, N,
                           slots, num_slots);
    trace("conv_tail_kernel<%s> grid=(%u,%u) block=%d lds=0", dt == KDA_BF16 ? "bf16" : "f32", grid.x,
          grid.y, kConvThreads);
    return hipGetLastError();
}

}  // namespace kda
