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

template <typename T>
__global__ void __launch_bounds__(kConvThreads)
conv_tail_kernel(const T *__restrict__ s0p, const T *__restrict__ s1p, const T *__restrict__ s2p,
                 int c0, int c1, int c2, int64_t total, const T *cs_in, T *cs_out,
                 const int32_t *__restrict__ cu, int num_seqs) {
    const int CC = c0 + c1 + c2;
    const int c = blockIdx.y * kConvThreads + threadIdx.x;
    const int n = blockIdx.x;
    if (c >= CC) return;
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
        else if (cs_in) vals[s] = cs_in[((int64_t)n * 3 + (3 + p)) * CC + c];
        else vals[s] = from_f32<T>(0.f);
    }
    // every thread reads its own (n, c) slots before writing them: in place is safe
#pragma unroll
    for (int s = 0; s < 3; ++s) cs_out[((int64_t)n * 3 + s) * CC + c] = vals[s];
}

template <typename T>
static hipError_t short_conv_t(const void *x, void *y, int64_t T_, int C, const float *w,
                               const float *b, const void *cs_in, const int32_t *cu, int N,
                               bool silu, hipStream_t s) {
    if (T_ == 0) return hipSuccess;
    // tokens on x (up to 2^31 blocks), channel pairs on y
    dim3 grid((unsigned)((T_ + kConvTokens - 1) / kConvTokens),
              (unsigned)(((C + 1) / 2 + kConvThreads - 1) / kConvThreads));
    if (silu)
        hipLaunchKernelGGL((short_conv_kernel<T, true>), grid, dim3(kConvThreads), 0, s,
                           (const T *)x, (T *)y, T_, C, w, b, (const T *)cs_in, cu, N);
    else
        hipLaunchKernelGGL((short_conv_kernel<T, false>), grid, dim3(kConvThreads), 0, s,
                           (const T *)x, (T *)y, T_, C, w, b, (const T *)cs_in, cu, N);
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
                            hipStream_t s) {
    const int CC = ch[0] + ch[1] + ch[2];
    dim3 grid((unsigned)N, (unsigned)((CC + kConvThreads - 1) / kConvThreads));
    if (dt == KDA_BF16)
        hipLaunchKernelGGL((conv_tail_kernel<__bf16>), grid, dim3(kConvThreads), 0, s,
                           (const __bf16 *)src[0], (const __bf16 *)src[1], (const __bf16 *)src[2],
                           ch[0], ch[1], ch[2], T_, (const __bf16 *)cs_in, (__bf16 *)cs_out, cu, N);
    else
        hipLaunchKernelGGL((conv_tail_kernel<float>), grid, dim3(kConvThreads), 0, s,
                           (const float *)src[0], (const float *)src[1], (const float *)src[2],
                           ch[0], ch[1], ch[2], T_, (const float *)cs_in, (float *)cs_out, cu, N);
    return hipGetLastError();
}

}  // namespace kda
