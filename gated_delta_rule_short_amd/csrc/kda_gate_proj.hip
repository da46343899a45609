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
// workgroup owns 64 tokens, every column and one quarter of K.  Two producer
// waves stream 64-wide K slabs of the token rows and the weight rows into a
// three-slab LDS ring with LDS-DMA (whole 128-byte row segments); eight compute
// waves, each 32 tokens x a quarter of the columns, read their MFMA fragments
// from the ring.  Reading the weights once per 64 tokens, in whole lines, is
// what bounds this product.  The quarters' fp32 partials go to the workspace and
// zreduce_kernel sums them in K order into z (bf16) and the finished beta.
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
constexpr int kSplit = 4;    // K ranges of the first product (one per workgroup)
constexpr int kMT = 64;      // tokens per zproj workgroup
constexpr int kSlabK = 64;   // K values per LDS slab: one 128-byte row segment
constexpr int kRing = 3;     // slabs in the ring (two in flight ahead of the MFMAs)

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

struct ZParams {
    const __bf16 *x, *w_a, *w_beta;
    float *part;  // [kSplit][T][N1] fp32 partial products (workspace)
    int64_t T;
    int hid, H;
};

// Slab rows: kMT token rows, then the N1 weight rows (W_a, then W_beta), 128 bytes
// each.  16-byte chunk c of row r sits at chunk c ^ (r & 7) of its LDS row, so the
// 16 rows one fragment read touches fall in different banks.
template <int NT>
struct ZGeom {
    static constexpr int N1 = 16 * NT, ROWS = kMT + N1;
    static constexpr int SLAB = ROWS * 128;           // bytes
    static constexpr int INST = SLAB / 1024;          // 1 KiB DMA instructions per slab
    static constexpr int LDS = kRing * SLAB;
    static constexpr int PW = 2;                      // producer waves
    static_assert(SLAB % 1024 == 0 && INST % PW == 0, "whole DMA instructions per producer");
    static_assert(INST / PW * (kRing - 1) < 64, "vmcnt range");
};

template <int NT>
__device__ __forceinline__ void zproj_issue(unsigned char *slot, const ZParams &p, int64_t t0, int k0,
                                            int pw, int lane) {
    typedef ZGeom<NT> G;
#pragma unroll
    for (int i = pw; i < G::INST; i += G::PW) {
        const int row = 8 * i + (lane >> 3), gc = (lane & 7) ^ (row & 7);
        const __bf16 *src;
        if (row < kMT) {
            int64_t t = t0 + row;
            t = t < p.T ? t : p.T - 1;
            src = p.x + t * p.hid;
        } else {
            const int n = row - kMT;
            src = n < kRank ? p.w_a + (size_t)n * p.hid : p.w_beta + (size_t)(n - kRank) * p.hid;
        }
        __builtin_amdgcn_global_load_lds(src + k0 + 8 * gc, (lds_void *)(slot + i * 1024), 16, 0, 0);
    }
}

template <int NT>
__global__ void __launch_bounds__(640) zproj_kernel(ZParams p) {
    typedef ZGeom<NT> G;
    constexpr int N1 = G::N1, PER = G::INST / G::PW;
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t t0 = (int64_t)blockIdx.x * kMT;
    const int kq = p.hid / kSplit, kb = blockIdx.y * kq;
    const int nsl = kq / kSlabK;

    if (wave >= 8) {
        // producers: slab s + 2 goes into the slot slab s - 1 used, once every
        // compute wave has passed barrier B_s (and so finished slab s - 1); bare
        // barriers, since a fence would drain the DMA in flight
        const int pw = wave - 8;
        zproj_issue<NT>(ring, p, t0, kb, pw, lane);
        if (nsl > 1) zproj_issue<NT>(ring + G::SLAB, p, t0, kb + kSlabK, pw, lane);
        for (int s = 0; s < nsl; ++s) {
            if (s + 1 < nsl) wait_vmcnt<PER>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();  // B_s: slab s in LDS
            if (s + 2 < nsl)
                zproj_issue<NT>(ring + ((s + 2) % kRing) * G::SLAB, p, t0, kb + (s + 2) * kSlabK, pw, lane);
        }
        return;
    }

    // compute wave: 32 tokens (half mh) x 16 NT / 4 columns (quarter nq)
    constexpr int NJ = NT / 4;
    static_assert(NT % 4 == 0, "column quarters of whole 16-column tiles");
    const int mh = wave & 1, nq = wave >> 1;
    const int m16 = lane & 15, g = lane >> 4;
    f32x4 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int arow[2], brow[NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i) arow[i] = 32 * mh + 16 * i + m16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) brow[j] = kMT + 16 * NJ * nq + 16 * j + m16;
    auto frag = [&](const unsigned char *slot, int row, int chunk) {
        return *reinterpret_cast<const bf16x8 *>(slot + row * 128 + ((chunk ^ (row & 7)) << 4));
    };
    for (int s = 0; s < nsl; ++s) {
        // B_s, with LDS fences: no fragment read moves across it (these waves have
        // no DMA of their own in flight, so the fences wait for nothing else)
        barrier_lds();
        const unsigned char *slot = ring + (s % kRing) * G::SLAB;
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // the slab's two k-steps of 32
            bf16x8 a[2], b[NJ];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = frag(slot, arow[i], 4 * h + g);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = frag(slot, brow[j], 4 * h + g);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mma_k32(a[i], b[j], acc[i][j]);
        }
    }
    // this K range's partial products (lane: rows 4 g + e of each 16-row block, column m16)
    float *part = p.part + (size_t)blockIdx.y * p.T * N1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t t = t0 + 32 * mh + 16 * i + 4 * g + e;
            if (t < p.T) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) part[t * N1 + 16 * NJ * nq + 16 * j + m16] = acc[i][j][e];
            }
        }
}

// The kSplit partials summed in K order: z (bf16) and beta = sigmoid.
__global__ void __launch_bounds__(256) zreduce_kernel(const float *part, __bf16 *z, __bf16 *beta,
                                                      int64_t T, int H) {
    const int N1 = kRank + H;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * N1) return;
    const int64_t t = idx / N1;
    const int n = (int)(idx - t * N1);
    const size_t sz = (size_t)T * N1;
    float y = part[idx];
#pragma unroll
    for (int q = 1; q < kSplit; ++q) y += part[q * sz + idx];
    if (n < kRank)
        z[t * kRank + n] = (__bf16)y;
    else
        beta[t * H + (n - kRank)] = (__bf16)sigmoidf_dev(y);
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
    typedef ZGeom<NT> G;
    static_assert(G::LDS <= 160 * 1024, "LDS budget");
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&zproj_kernel<NT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
    });
    if (attr != hipSuccess) return attr;
    const dim3 grid((unsigned)((zp.T + kMT - 1) / kMT), kSplit);
    hipLaunchKernelGGL(zproj_kernel<NT>, grid, dim3(640), G::LDS, s, zp);
    trace("zproj_kernel<%d> grid=(%u,%u) block=640 lds=%d", NT, grid.x, grid.y, (int)G::LDS);
    return hipGetLastError();
}

}  // namespace

size_t gate_proj_workspace_bytes(int64_t T, int H) {
    // fp32 partials of the first product, then z (bf16)
    return (size_t)kSplit * (size_t)T * (size_t)(kRank + H) * sizeof(float) + (size_t)T * kRank * sizeof(__bf16);
}

hipError_t launch_gate_proj(const kda_gate_beta_args *a, hipStream_t s) {
    const int64_t T = a->total_tokens;
    if (T == 0) return hipSuccess;
    const int H = a->num_heads, N1 = kRank + H;
    ZParams zp;
    zp.x = static_cast<const __bf16 *>(a->x);
    zp.w_a = static_cast<const __bf16 *>(a->w_a);
    zp.w_beta = static_cast<const __bf16 *>(a->w_beta);
    zp.part = static_cast<float *>(a->workspace);
    zp.T = T; zp.hid = a->hidden; zp.H = H;
    __bf16 *z = reinterpret_cast<__bf16 *>(zp.part + (size_t)kSplit * T * N1);
    hipError_t e;
    switch (N1 / 16) {
        case 12: e = launch_zproj<12>(zp, s); break;
        default: e = launch_zproj<16>(zp, s); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zreduce_kernel, dim3((unsigned)((T * N1 + 255) / 256)), dim3(256), 0, s, zp.part, z,
                       static_cast<__bf16 *>(a->beta), T, H);
    trace("zreduce_kernel grid=(%u) block=256 lds=0", (unsigned)((T * N1 + 255) / 256));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    EParams ep;
    ep.z = z;
    ep.w_b = static_cast<const __bf16 *>(a->w_b);
    ep.gate = static_cast<__bf16 *>(a->gate);
    ep.T = T; ep.hd = H * kHeadDim;
    ep.lb = a->gate_lower_bound;
    ep.glog = (a->flags & KDA_F_GATE_IS_LOG) ? 1 : 0;
    const dim3 g2((unsigned)((T + 63) / 64), (unsigned)(ep.hd / (256 * kCT)));
    hipLaunchKernelGGL(gate_expand_kernel, g2, dim3(256), 0, s, ep);
    trace("gate_expand_kernel grid=(%u,%u) block=256", g2.x, g2.y);
    return hipGetLastError();
}

}  // namespace kda
