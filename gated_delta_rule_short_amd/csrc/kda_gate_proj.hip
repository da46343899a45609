// kda_gate_proj.hip -- the gate and beta in-projections of a KDA layer, with
// their activations fused into the matrix-core epilogues.
//
// Source: "GLM-5.3-Flash Internals" (Zek-Takai dataset card): the decoder's
// hidden width is 4096 (section "Anatomy"), and its activation batteries name
// the KDA gate projections ("KDA gate_proj", "g_b_proj": the second factor of a
// two-factor gate projection).  "GLM-5.3-Flash im Detail", section
// "Sequenz-Mixing": a channel-wise forget gate with log-decay >= -5 and a
// scalar beta per head and token.  Per token x (hidden wide):
//     z    = W_a x            (rank r = 128)
//     a    = W_b z            (H * dk gate channels, head-major)
//     g    = lb * sigmoid(a)  (written instead of a with KDA_F_GATE_IS_LOG)
//     beta = sigmoid(W_beta x)
//
// zproj_kernel: y = x [W_a; W_beta]^T, N = r + H columns, K = hidden.  A
// workgroup owns 16 tokens and every column; its four waves take one quarter of
// K each (both operands are K-contiguous rows, the order the 16x16x32 bf16 MFMA
// reads, fetched from L2 three k-steps ahead) and add their partial tiles in LDS.
// The sums leave as z (bf16, the workspace) and as the finished beta.
//
// gate_expand_kernel: per 64 tokens x 256 gate channels, z (from the workspace,
// via LDS) times W_b (K = 128) with MFMA, the gate activation, the tile staged
// in LDS and written as whole 512-byte rows.
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kRank = 128;   // r
constexpr int kZT = 16;      // tokens per zproj workgroup

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

struct ZParams {
    const __bf16 *x, *w_a, *w_beta;
    __bf16 *z, *beta;  // z [T][r] (workspace), beta [T][H]
    int64_t T;
    int hid, H;
};

template <int NT>  // 16-column tiles: (r + H) / 16
__global__ void __launch_bounds__(256) zproj_kernel(ZParams p) {
    constexpr int N1 = 16 * NT;
    constexpr int PF = 3;  // k-steps of fragments in flight ahead of the MFMAs
    extern __shared__ __attribute__((aligned(16))) float red[];  // [4 waves][kZT][N1]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m16 = lane & 15, k8 = (lane >> 4) * 8;
    const int64_t t0 = (int64_t)blockIdx.x * kZT;
    const int kq = p.hid / 4, kb = wave * kq;  // this wave's quarter of K
    const int steps = kq / 32;
    int64_t t = t0 + m16;
    t = t < p.T ? t : p.T - 1;
    const __bf16 *xr = p.x + t * p.hid + kb + k8;
    const __bf16 *wr[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = 16 * j + m16;
        wr[j] = (n < kRank ? p.w_a + (size_t)n * p.hid : p.w_beta + (size_t)(n - kRank) * p.hid) + kb + k8;
    }
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // a ring of PF k-steps of fragments: step s sits in slot s % PF
    bf16x8 a[PF], b[PF][NT];
#pragma unroll
    for (int q = 0; q < PF; ++q)
        if (q < steps) {
            a[q] = ld8(xr + 32 * q);
#pragma unroll
            for (int j = 0; j < NT; ++j) b[q][j] = ld8(wr[j] + 32 * q);
        }
    for (int s0 = 0; s0 < steps; s0 += PF) {
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int st = s0 + q;
            if (st < steps) {
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[j] = mma_k32(a[q], b[q][j], acc[j]);
                if (st + PF < steps) {  // refill the slot just consumed
                    a[q] = ld8(xr + 32 * (st + PF));
#pragma unroll
                    for (int j = 0; j < NT; ++j) b[q][j] = ld8(wr[j] + 32 * (st + PF));
                }
            }
        }
    }
    // partial tile of this wave into LDS (lane: rows 4 (lane / 16) + e, column m16)
    float *mine = red + wave * kZT * N1;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < NT; ++j) mine[(4 * (lane >> 4) + e) * N1 + 16 * j + m16] = acc[j][e];
    __syncthreads();
    // the four quarters summed in K order; z rounded to bf16, beta through the sigmoid
    for (int idx = tid; idx < kZT * N1; idx += 256) {
        const int r = idx / N1, n = idx - r * N1;
        const int64_t tt = t0 + r;
        if (tt >= p.T) continue;
        const float y = ((red[idx] + red[kZT * N1 + idx]) + red[2 * kZT * N1 + idx]) + red[3 * kZT * N1 + idx];
        if (n < kRank)
            p.z[tt * kRank + n] = (__bf16)y;
        else
            p.beta[tt * p.H + (n - kRank)] = (__bf16)sigmoidf_dev(y);
    }
}

struct EParams {
    const __bf16 *z, *w_b;
    __bf16 *gate;
    int64_t T;
    int hd;  // H * dk gate channels
    float lb;
    int glog;
};

constexpr int kZS = kRank + 8;    // LDS row stride of z (bf16 elements)
constexpr int kOS = 256 + 8;      // LDS row stride of the output tile

__global__ void __launch_bounds__(256) gate_expand_kernel(EParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 zs[64 * kZS];
    __shared__ __attribute__((aligned(16))) __bf16 os[64 * kOS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m16 = lane & 15, k8 = (lane >> 4) * 8;
    const int64_t t0 = (int64_t)blockIdx.x * 64;
    const int c0 = blockIdx.y * 256;
    // this wave's W_b fragments (64 channels c0 + 64 wave .., all of K = 128), in
    // flight while z is staged
    const __bf16 *wb = p.w_b + (size_t)(c0 + 64 * wave + m16) * kRank + k8;
    bf16x8 bw[kRank / 32][4];
#pragma unroll
    for (int kk = 0; kk < kRank / 32; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) bw[kk][j] = ld8(wb + (size_t)16 * j * kRank + 32 * kk);
    // z rows of the 64 tokens (the last one repeated past T): 16 pieces of 16 B per row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int piece = q * 256 + tid, r = piece >> 4, c = (piece & 15) * 8;
        int64_t t = t0 + r;
        t = t < p.T ? t : p.T - 1;
        *reinterpret_cast<bf16x8 *>(zs + r * kZS + c) = ld8(p.z + t * kRank + c);
    }
    __syncthreads();
    // this wave: all 64 tokens x 64 channels c0 + 64 wave ..
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kRank / 32; ++kk) {
        bf16x8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = ld8(zs + (16 * i + m16) * kZS + 32 * kk + k8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mma_k32(a[i], bw[kk][j], acc[i][j]);
    }
    // epilogue: the gate activation, then the tile transposed to rows in LDS
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = p.glog ? p.lb * sigmoidf_dev(acc[i][j][e]) : acc[i][j][e];
                os[(16 * i + 4 * (lane >> 4) + e) * kOS + 64 * wave + 16 * j + m16] = (__bf16)v;
            }
    __syncthreads();
    // 64 rows of 512 bytes, 16 bytes per lane
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int piece = q * 256 + tid, r = piece >> 5, c = (piece & 31) * 8;
        const int64_t t = t0 + r;
        if (t < p.T)
            *reinterpret_cast<bf16x8 *>(p.gate + t * p.hd + c0 + c) =
                *reinterpret_cast<const bf16x8 *>(os + r * kOS + c);
    }
}

template <int NT>
static hipError_t launch_zproj(const ZParams &zp, hipStream_t s) {
    constexpr int lds = 4 * kZT * 16 * NT * (int)sizeof(float);
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&zproj_kernel<NT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(zproj_kernel<NT>, dim3((unsigned)((zp.T + kZT - 1) / kZT)), dim3(256), lds, s, zp);
    return hipGetLastError();
}

}  // namespace

size_t gate_proj_workspace_bytes(int64_t T, int H) {
    (void)H;
    return (size_t)T * kRank * sizeof(__bf16);  // z
}

hipError_t launch_gate_proj(const kda_gate_beta_args *a, hipStream_t s) {
    const int64_t T = a->total_tokens;
    if (T == 0) return hipSuccess;
    const int H = a->num_heads;
    ZParams zp;
    zp.x = static_cast<const __bf16 *>(a->x);
    zp.w_a = static_cast<const __bf16 *>(a->w_a);
    zp.w_beta = static_cast<const __bf16 *>(a->w_beta);
    zp.z = static_cast<__bf16 *>(a->workspace);
    zp.beta = static_cast<__bf16 *>(a->beta);
    zp.T = T; zp.hid = a->hidden; zp.H = H;
    hipError_t e;
    switch ((kRank + H) / 16) {
        case 10: e = launch_zproj<10>(zp, s); break;
        case 12: e = launch_zproj<12>(zp, s); break;
        case 14: e = launch_zproj<14>(zp, s); break;
        default: e = launch_zproj<16>(zp, s); break;
    }
    if (e != hipSuccess) return e;
    EParams ep;
    ep.z = zp.z;
    ep.w_b = static_cast<const __bf16 *>(a->w_b);
    ep.gate = static_cast<__bf16 *>(a->gate);
    ep.T = T; ep.hd = H * kHeadDim;
    ep.lb = a->gate_lower_bound;
    ep.glog = (a->flags & KDA_F_GATE_IS_LOG) ? 1 : 0;
    const dim3 g2((unsigned)((T + 63) / 64), (unsigned)(ep.hd / 256));
    hipLaunchKernelGGL(gate_expand_kernel, g2, dim3(256), 0, s, ep);
    return hipGetLastError();
}

}  // namespace kda
