// kda_decode.hip -- single-token recurrent update of the KDA state.
//
// Source: "GLM-5.3-Flash im Detail" (flozi.net), section "Sequenz-Mixing":
// decoding one token is a recurrent update of the per-head matrix state (fp32,
// dk x dv = 128 x 128); conv of width four on q, k, v; channel-wise forget gate
// with log-decay >= -5; scalar-beta delta-rule write; the query reads the
// updated state.
//
// One workgroup of 256 threads per (sequence, head).  The step is bound by HBM:
// the 64 KiB state is read once and written once.  Thread t owns columns
// 4*(t%32)..+3 of rows (t/32) + 8*m, m = 0..15: every load instruction of the
// workgroup covers eight whole 512-byte rows (fully coalesced float4 accesses),
// and the 64 state values stay in registers between the read and the write.
// The state loads are issued before the conv / L2 / gate prologue, so the
// prologue runs under the memory latency.  Per column j with decayed rows
// S'_i = alpha_i S_i:
//     a_j = sum_i S'_ij k_i,  c_j = sum_i S'_ij q_i
//     u_j = beta (v_j - a_j), o_j = scale (c_j + u_j (k . q)), S_ij = S'_ij + k_i u_j
// The row sums reduce across the two row groups of a wave (lane xor 32) and
// across the four waves through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

struct DecodeParams {
    const void *q, *k, *v, *gate, *beta;
    const float *w, *bias;
    void *cs;
    float *state;
    void *o;
    int H;
    float scale, lb;
    uint32_t flags;
};

template <typename T>
__global__ void __launch_bounds__(256) decode_kernel(DecodeParams p) {
    constexpr int D = kHeadDim;
    const int pr = blockIdx.x;
    const int H = p.H;
    const int n = pr / H, h = pr - n * H;
    const int tid = threadIdx.x;
    const int cg = tid & 31, rg = tid >> 5, wave = tid >> 6;

    __shared__ __attribute__((aligned(16))) float s_q[D], s_k[D], s_v[D], s_alpha[D];
    __shared__ float s_red[2][3];
    __shared__ f32x4 s_part[4][32][2];

    // 1. issue the state loads (independent of the prologue).  The state is
    // streamed exactly once each way: non-temporal loads and stores keep it from
    // displacing the small, reused operands in L2.
    float *S = p.state + (size_t)pr * D * D;
    f32x4 st[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        st[m] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(S + (size_t)(rg + 8 * m) * D + 4 * cg));

    // 2. prologue: conv (and cache shift), L2 of q and k, gate
    const int CC = 3 * H * D;
    T *cs = reinterpret_cast<T *>(p.cs) + (size_t)n * 3 * CC;
    const bool silu = p.flags & KDA_F_SILU;
    const bool l2 = !(p.flags & KDA_F_NO_QK_L2NORM);
    const bool glog = p.flags & KDA_F_GATE_IS_LOG;
    const size_t tok = (size_t)pr * D;  // offset of this (sequence, head) row
    auto conv = [&](const T *x, int ch) -> float {
        const float raw = to_f32(x[tok + (ch % D)]);
        const float h0 = to_f32(cs[ch]), h1 = to_f32(cs[CC + ch]), h2 = to_f32(cs[2 * CC + ch]);
        const float *wc = p.w + 4 * ch;
        float y = (p.bias ? p.bias[ch] : 0.f) + wc[0] * h0 + wc[1] * h1 + wc[2] * h2 + wc[3] * raw;
        // shift the cache by one token (this workgroup alone owns these channels)
        cs[ch] = cs[CC + ch];
        cs[CC + ch] = cs[2 * CC + ch];
        cs[2 * CC + ch] = from_f32<T>(raw);
        if (silu) y = y * sigmoidf_dev(y);
        return y;
    };
    float part_qq = 0.f, part_kk = 0.f, part_qk = 0.f;
    if (tid < D) {
        const int c = tid;
        const float qc = conv(reinterpret_cast<const T *>(p.q), h * D + c);
        const float kc = conv(reinterpret_cast<const T *>(p.k), H * D + h * D + c);
        s_q[c] = qc;
        s_k[c] = kc;
        part_qq = qc * qc;
        part_kk = kc * kc;
        part_qk = qc * kc;
    } else {
        const int c = tid - D;
        s_v[c] = conv(reinterpret_cast<const T *>(p.v), 2 * H * D + h * D + c);
        const float a = to_f32(reinterpret_cast<const T *>(p.gate)[tok + c]);
        const float g = glog ? fmaxf(a, p.lb) : p.lb * sigmoidf_dev(a);
        s_alpha[c] = __expf(g);
    }
    if (wave < 2) {
        part_qq = wave_sum(part_qq);
        part_kk = wave_sum(part_kk);
        part_qk = wave_sum(part_qk);
        if ((tid & 63) == 0) {
            s_red[wave][0] = part_qq;
            s_red[wave][1] = part_kk;
            s_red[wave][2] = part_qk;
        }
    }
    __syncthreads();
    const float sqq = s_red[0][0] + s_red[1][0];
    const float skk = s_red[0][1] + s_red[1][1];
    const float sqk = s_red[0][2] + s_red[1][2];
    const float iq = l2 ? rsqrtf(sqq + 1e-6f) : 1.f;
    const float ik = l2 ? rsqrtf(skk + 1e-6f) : 1.f;
    const float kq = sqk * iq * ik;
    const float beta = to_f32(reinterpret_cast<const T *>(p.beta)[pr]);

    // 3. decay the rows and reduce S'^T k and S'^T q over this thread's 16 rows
    f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
    float krow[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int r = rg + 8 * m;
        const float al = s_alpha[r];
        const float kr = s_k[r] * ik;
        const float qr = s_q[r] * iq;
        krow[m] = kr;
        st[m] *= al;
        ak += st[m] * kr;
        aq += st[m] * qr;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ak[e] += __shfl_xor(ak[e], 32, kWave);
        aq[e] += __shfl_xor(aq[e], 32, kWave);
    }
    if ((tid & 63) < 32) {
        s_part[wave][cg][0] = ak;
        s_part[wave][cg][1] = aq;
    }
    __syncthreads();
    f32x4 sk = s_part[0][cg][0] + s_part[1][cg][0] + s_part[2][cg][0] + s_part[3][cg][0];
    f32x4 sq = s_part[0][cg][1] + s_part[1][cg][1] + s_part[2][cg][1] + s_part[3][cg][1];

    // 4. delta-rule value, output, write-back
    f32x4 vv = *reinterpret_cast<const f32x4 *>(&s_v[4 * cg]);
    f32x4 u = beta * (vv - sk);
    if (rg == 0) {
        f32x4 ov = p.scale * (sq + u * kq);
        T *o = reinterpret_cast<T *>(p.o) + tok + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(ov[e]);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        st[m] += krow[m] * u;
        __builtin_nontemporal_store(st[m], reinterpret_cast<f32x4 *>(S + (size_t)(rg + 8 * m) * D + 4 * cg));
    }
}

hipError_t launch_decode(const kda_decode_args *a, hipStream_t s) {
    DecodeParams p;
    p.q = a->q; p.k = a->k; p.v = a->v; p.gate = a->gate; p.beta = a->beta;
    p.w = a->conv_weight; p.bias = a->conv_bias;
    p.cs = a->conv_state; p.state = a->state; p.o = a->o;
    p.H = a->num_heads;
    p.scale = a->scale; p.lb = a->gate_lower_bound; p.flags = a->flags;
    const unsigned blocks = (unsigned)a->num_seqs * (unsigned)a->num_heads;
    if (a->dtype == KDA_BF16)
        hipLaunchKernelGGL(decode_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(decode_kernel<float>, dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
