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
// workgroup owns 32 tokens and every column; its eight waves take one column half
// and one K quarter each (both operands are K-contiguous rows, the order the
// 16x16x32 bf16 MFMA reads; a lane's two k-steps of a super-step read one whole
// 128-byte line of a row, fetched a super-step ahead), and the K quarters add
// their tiles through LDS in K order.
// The sums leave as z (bf16, the workspace) and as the finished beta.
//
// gate_expand_kernel: per 64 tokens x 1024 gate channels (four tiles of 256),
// z (from the workspace, via LDS) times W_b (K = 128) with MFMA, the gate
// activation, each tile staged in LDS and written as whole 512-byte rows; the
// next tile's weights load while a tile is written.
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kRank = 128;   // r
constexpr int kZT = 32;      // tokens per zproj workgroup

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

struct ZParams {
    const __bf16 *x, *w_a, *w_beta;
    __bf16 *z, *beta;  // z [T][r] (workspace), beta [T][H]
    int64_t T;
    int hid, H;
};

template <int NT>  // 16-column tiles: (r + H) / 16, even
__global__ void __launch_bounds__(512) zproj_kernel(ZParams p) {
    constexpr int N1 = 16 * NT, NTW = NT / 2;  // columns, column tiles per wave
    extern __shared__ __attribute__((aligned(16))) float red[];  // [3 K quarters][2 halves][kZT][N1 / 2]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m16 = lane & 15, g = lane >> 4;
    const int wn = wave & 1, wk = wave >> 1;  // column half, K quarter
    const int64_t t0 = (int64_t)blockIdx.x * kZT;
    const int kh = p.hid / 4, kb = wk * kh;
    const int steps = kh / 64;  // super-steps of 64 K values: one 128-byte line per row
    // In super-step u, k-step h (0, 1) lane group g covers K values
    // kb + 64 u + 16 g + 8 h .. + 7 of both operands: the two k-steps of a row read
    // one whole line, back to back.  (Any K order gives the same sums as long as
    // both operands use it.)
    const __bf16 *xr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t t = t0 + 16 * i + m16;
        t = t < p.T ? t : p.T - 1;
        xr[i] = p.x + t * p.hid + kb + 16 * g;
    }
    const __bf16 *wr[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int n = wn * 16 * NTW + 16 * j + m16;
        wr[j] = (n < kRank ? p.w_a + (size_t)n * p.hid : p.w_beta + (size_t)(n - kRank) * p.hid) + kb + 16 * g;
    }
    f32x4 acc[2][NTW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a[2][2], b[2][NTW];  // [k-step h][...]
    auto load = [&](int u, bf16x8 (&la)[2][2], bf16x8 (&lb)[2][NTW]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) la[h][i] = ld8(xr[i] + 64 * u + 8 * h);
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) lb[h][j] = ld8(wr[j] + 64 * u + 8 * h);
    };
    load(0, a, b);
    for (int u = 0; u < steps; ++u) {
        bf16x8 an[2][2], bn[2][NTW];
        if (u + 1 < steps) load(u + 1, an, bn);  // in flight during this super-step's MFMAs
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[i][j] = mma_k32(a[h][i], b[h][j], acc[i][j]);
        if (u + 1 < steps) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < 2; ++i) a[h][i] = an[h][i];
#pragma unroll
                for (int j = 0; j < NTW; ++j) b[h][j] = bn[h][j];
            }
        }
    }
    // K quarters 1..3 hand their tiles to quarter 0 through LDS (lane: rows
    // 4 g + e of each 16-row block, column m16)
    constexpr int HW = N1 / 2, TILE = kZT * HW;
    if (wk > 0) {
        float *mine = red + ((wk - 1) * 2 + wn) * TILE;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int j = 0; j < NTW; ++j) mine[(16 * i + 4 * g + e) * HW + 16 * j + m16] = acc[i][j][e];
    }
    barrier_lds();
    if (wk > 0) return;
    const float *q1 = red + wn * TILE, *q2 = red + (2 + wn) * TILE, *q3 = red + (4 + wn) * TILE;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * i + 4 * g + e;
            const int64_t t = t0 + r;
            if (t >= p.T) continue;
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int n = wn * HW + 16 * j + m16;
                const int at = r * HW + 16 * j + m16;
                const float y = ((acc[i][j][e] + q1[at]) + q2[at]) + q3[at];  // K order
                if (n < kRank)
                    p.z[t * kRank + n] = (__bf16)y;
                else
                    p.beta[t * p.H + (n - kRank)] = (__bf16)sigmoidf_dev(y);
            }
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

constexpr int kCT = 4;  // 256-channel tiles per gate_expand workgroup

__global__ void __launch_bounds__(256) gate_expand_kernel(EParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 zs[64 * kZS];
    __shared__ __attribute__((aligned(16))) __bf16 os[64 * kOS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m16 = lane & 15, k8 = (lane >> 4) * 8;
    const int64_t t0 = (int64_t)blockIdx.x * 64;
    const int cbase = blockIdx.y * (256 * kCT);
    // this wave's W_b fragments for channel tile ct: channels cbase + 256 ct +
    // 64 wave .., all of K = 128
    bf16x8 bw[kRank / 32][4];
    auto load_w = [&](int ct) {
        const __bf16 *wb = p.w_b + (size_t)(cbase + 256 * ct + 64 * wave + m16) * kRank + k8;
#pragma unroll
        for (int kk = 0; kk < kRank / 32; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) bw[kk][j] = ld8(wb + (size_t)16 * j * kRank + 32 * kk);
    };
    load_w(0);
    // z rows of the 64 tokens (the last one repeated past T): 16 pieces of 16 B per row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int piece = q * 256 + tid, r = piece >> 4, c = (piece & 15) * 8;
        int64_t t = t0 + r;
        t = t < p.T ? t : p.T - 1;
        *reinterpret_cast<bf16x8 *>(zs + r * kZS + c) = ld8(p.z + t * kRank + c);
    }
    barrier_lds();  // LDS only: the weight loads stay in flight
    for (int ct = 0; ct < kCT; ++ct) {
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
        if (ct + 1 < kCT) load_w(ct + 1);  // next tile's weights, in flight during the epilogue
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
        barrier_lds();
        // 64 rows of 512 bytes, 16 bytes per lane
        const int c0 = cbase + 256 * ct;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int piece = q * 256 + tid, r = piece >> 5, c = (piece & 31) * 8;
            const int64_t t = t0 + r;
            if (t < p.T)
                *reinterpret_cast<bf16x8 *>(p.gate + t * p.hd + c0 + c) =
                    *reinterpret_cast<const bf16x8 *>(os + r * kOS + c);
        }
        barrier_lds();  // the next tile's epilogue rewrites os (stores stay in flight)
    }
}

template <int NT>
static hipError_t launch_zproj(const ZParams &zp, hipStream_t s) {
    constexpr int lds = 3 * kZT * 16 * NT * (int)sizeof(float);  // three K quarters' tiles
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&zproj_kernel<NT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(zproj_kernel<NT>, dim3((unsigned)((zp.T + kZT - 1) / kZT)), dim3(512), lds, s, zp);
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
    const dim3 g2((unsigned)((T + 63) / 64), (unsigned)(ep.hd / (256 * kCT)));
    hipLaunchKernelGGL(gate_expand_kernel, g2, dim3(256), 0, s, ep);
    return hipGetLastError();
}

}  // namespace kda
