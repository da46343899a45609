// kda_prefill_split.hip -- two-pass KDA prefill with 16-token sub-chunks.
//
// Source: "GLM-5.3-Flash im Detail" (flozi.net), section "Sequenz-Mixing":
// in prefill the tokens inside chunks are evaluated in parallel while a state
// is handed from chunk to chunk.  Per head: width-4 causal conv of q, k, v,
// channel-wise forget gate (log-decay >= -5), scalar-beta delta-rule write into
// a 128 x 128 fp32 state, query read of the updated state.
//
// Pass A (intra_kernel) is parallel over (head, 64-token block): each wave takes
// one 16-token sub-chunk of one sequence and computes, relative to the state on
// entry to the sub-chunk,
//     A = strict_lower(K~ K^T . decay),  P = lower(Q~ K^T . decay),
//     X = (I + diag(beta) A)^-1,  W = X diag(beta) (K . 2^b),  U0 = X diag(beta) V,
// with b the log2-decay cumsum from the sub-chunk start (>= -115.4, so every
// factor is a finite fp32/bf16 number), and writes them as matrix-core
// fragments to a workspace record.  Pass B (scan_kernel) runs one workgroup per
// (sequence, head, dv tile) over its sub-chunks in order:
//     U = U0 - W S,  O = scale ((Q . 2^b) S + P U),
//     S = diag(2^b_last) S + (K . 2^(b_last - b))^T U.
// Pass A does the conv / L2 / gate work once per token and head, over the
// whole GPU; pass B keeps the fp32 state in registers (accumulator layout) for
// the whole sequence and streams the records through an LDS ring filled by
// producer waves with LDS DMA, so several sub-chunks are in flight while
// the consumer waves run the recurrence.  The workspace costs extra HBM
// traffic (one 17 KiB record per sub-chunk and head, written once and read
// once), which pays off when there are too few (sequence, head) pairs to fill
// the GPU otherwise.
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mma.h"

// Producer waves of the pass-B workgroup (LDS DMA issue is per wave, so more
// waves deliver records faster; four measured best on gfx950).
#ifndef KDA_SCAN_PRODUCERS
#define KDA_SCAN_PRODUCERS 4
#endif

namespace kda {

namespace {

constexpr float kLog2eS = 1.4426950408889634f;

// Workspace record of one (head, sub-chunk), byte offsets; bf16 unless noted.
//   WN  [4][64][8]  -W, A-operand fragments (rows tokens, K = dk, permuted pairs)
//   QG  [4][64][8]  Q . 2^b, same fragment layout
//   KD  [8][64][4]  (K . 2^(b_last - b))^T, A-operand fragments (rows dk, K = tokens)
//   PP  [64][4]     P, A-operand fragment (rows tokens, K = tokens)
//   GAM [128] fp32  2^b_last per dk channel
//   U0  [8][64][4]  X diag(beta) V, accumulator layout (rows tokens, columns dv)
// Everything a workgroup of pass B shares comes first (R_U0 bytes), then the
// per-dv-tile U0 fragments, so each stage is two contiguous DMA ranges.
constexpr int R_WN = 0, R_QG = 4096, R_KD = 8192, R_PP = 12288, R_GAM = 12800, R_U0 = 13312;
constexpr size_t kRec = 17408;
static_assert(R_U0 % 1024 == 0, "shared part moves in whole DMA KiB");

struct SplitParams {
    const void *q, *k, *v, *gate, *beta;
    const float *w, *bias;
    const void *cs_in;
    const void *state_in;   // fp32, or bf16 when state_bf16
    void *state_out;
    int state_bf16;
    const int32_t *slots;   // pool row of each sequence (state, conv state), or null
    int num_slots;
    void *o;
    const int32_t *cu;
    unsigned char *ws;
    int64_t total, nslots;
    int num_seqs, H;
    float scale, lb;
    uint32_t flags;
    int pairs, tiles;
    int a_heads_fast;  // pass-A grid: heads in x (slot groups in y), else the reverse
    int64_t a_stride;  // pass A: slot distance between a wave's two tasks (4 x slot groups)
};

// Slot of sub-chunk j of sequence n (start s0): distinct for all (n, j) and
// below total/16 + num_seqs, with consecutive j in consecutive slots.
__device__ __forceinline__ int64_t sub_slot(int64_t s0, int64_t j, int n) { return (s0 + 16 * j) / 16 + n; }

// Per-wave LDS of pass A (bytes).  Row-major tiles hold A_SRM bf16 per token
// row, transposed tiles A_STR (A_VTS) bf16 per channel row.  beta V
// (transposed, VT) is formed after the QG export, in the then dead QL area.
constexpr int A_SRM = 132, A_STR = 20, A_VTS = 16;
constexpr int A_KL = 0, A_QL = A_KL + 16 * A_SRM * 2, A_KI = A_QL + 16 * A_SRM * 2;
constexpr int A_KGT = A_KI + 16 * A_SRM * 2, A_PS = A_KGT + 128 * A_STR * 2;
constexpr int A_WAVE = A_PS + 16 * A_STR * 2;
constexpr int A_VT = A_QL;
static_assert(A_WAVE % 16 == 0, "wave region alignment");
static_assert(128 * A_VTS * 2 <= 16 * A_SRM * 2, "VT fits in the QL area");
static_assert(8 * A_WAVE <= 163840, "two workgroups of four waves per CU");

typedef Ops<__bf16> OPB;

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf_ch(uint32_t u, int e) { return e ? bf_hi(u) : bf_lo(u); }

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Width-4 causal conv of 16 rows of this lane's two channels from 19 packed raw
// rows (the 3 history rows first), bias folded into the first tap.
__device__ __forceinline__ void conv16(const uint32_t (&x)[19], const float (&wt)[2][4],
                                       const float (&bs)[2], float (&y)[16][2]) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float a = fmaf(wt[e][0], bf_ch(x[rr], e), bs[e]);
            a = fmaf(wt[e][1], bf_ch(x[rr + 1], e), a);
            a = fmaf(wt[e][2], bf_ch(x[rr + 2], e), a);
            y[rr][e] = fmaf(wt[e][3], bf_ch(x[rr + 3], e), a);
        }
}

// Per-row 1 / sqrt(sum of squares + eps) over the 128 channels (two per lane; a
// wave-uniform value per row), or 1 without the L2 step.
__device__ __forceinline__ void l2_scale(const float (&y)[16][2], bool l2, int lane, float (&r)[16]) {
    if (!l2) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) r[rr] = 1.f;
        return;
    }
    float p[16], s4[4];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) p[rr] = fmaf(y[rr][0], y[rr][0], y[rr][1] * y[rr][1]);
    rows16_sum(p, s4, lane);
#pragma unroll
    for (int t = 0; t < 4; ++t) s4[t] = __builtin_amdgcn_rsqf(s4[t] + 1e-6f);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) r[rr] = row_value(s4, rr);
}

// One pass-A task: sub-chunk j (rows 16 j .. 16 j + 15) of sequence n, which
// starts at token s0 and holds L tokens.
struct SubTask {
    int64_t slot, s0, L, j;
    int n;
};

// Raw inputs of one sub-chunk for this lane's two channels, as packed bf16
// pairs: rows p0-3 .. p0+15 of q, k, v (clamped into the sequence; the three
// rows before a sequence come from the conv state or are zero) and rows p0 ..
// p0+15 of the gate; beta of row p0 + lane in lanes 0..15.  The gate, k and
// beta ("early") are needed first and are loaded one sub-chunk ahead; q and v
// ("late") are loaded when the sub-chunk starts.
struct EarlyRows {
    uint32_t xk[19], xa[16];
    uint32_t beta_bits;  // raw bf16 of beta (row clamped into the sequence); masked at use
};
struct LateRows {
    uint32_t xq[19], xv[19];
};

// Conv taps and bias of this lane's two q, k and v channels of head h.
struct ConvW {
    float w[3][2][4], b[3][2];
};

__device__ __forceinline__ void load_conv_w(const SplitParams &p, int h, int lane, ConvW &cw) {
    constexpr int D = kHeadDim;
    const int c0 = 2 * lane;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int ch = t * p.H * D + h * D + c0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(p.w + 4 * (ch + e));
#pragma unroll
            for (int i = 0; i < 4; ++i) cw.w[t][e][i] = a[i];
            cw.b[t][e] = p.bias ? p.bias[ch + e] : 0.f;
        }
    }
}

// Token rows of one sub-chunk as a buffer resource: rows p0-3 .. p0+15 of the
// sequence, clamped into it, starting at the first one used (all offsets are
// then small and non-negative).  Each lane reads its two channels (4 bytes at
// 4 * lane) of a row at a wave-uniform row offset, so no per-lane address
// arithmetic is needed.
// Sequence-relative rows are 32-bit (the token count is below 2^31), so the
// clamps are scalar compares rather than 64-bit vector ones.
struct RowWindow {
    int lo, hi, p0, L;  // first and last row used (sequence-relative), p0, length
};
__device__ __forceinline__ RowWindow row_window(const SubTask &tk, int first) {
    RowWindow w;
    w.p0 = 16 * (int)tk.j;
    w.L = (int)tk.L;
    int lo = w.p0 + first, hi = w.p0 + 15;
    lo = lo < 0 ? 0 : (lo >= w.L ? w.L - 1 : lo);
    hi = hi >= w.L ? w.L - 1 : hi;
    w.lo = lo;
    w.hi = hi;
    return w;
}
// Buffer resource over rows lo .. hi of this head's channels of tensor x (data
// format 32-bit, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *x, const SubTask &tk, int h,
                                                          const RowWindow &w, int64_t rowbytes) {
    const char *b = reinterpret_cast<const char *>(x) + (size_t)h * kHeadDim * 2 + (size_t)(tk.s0 + w.lo) * rowbytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(b), 0, (int)((w.hi - w.lo + 1) * rowbytes), 0x00020000);
}
// Byte offset of sub-chunk row r (-3 .. 15), clamped into the sequence, in the window.
__device__ __forceinline__ int row_soff(const RowWindow &w, int r, int rowbytes) {
    int sp = w.p0 + r;
    sp = sp < 0 ? 0 : (sp >= w.L ? w.L - 1 : sp);
    return (sp - w.lo) * rowbytes;
}

// The three rows before a sequence for tensor t (0 q, 1 k, 2 v): conv state or zeros.
__device__ __forceinline__ void load_history(const SplitParams &p, const SubTask &tk, int h, int lane, int t,
                                             uint32_t (&x)[19]) {
    constexpr int D = kHeadDim;
    const int CCH = 3 * p.H * D;
    const int ch = t * p.H * D + h * D + 2 * lane;
    const int slot = pool_slot(p.slots, p.num_slots, tk.n);
    const __bf16 *csn =
        p.cs_in && slot >= 0 ? reinterpret_cast<const __bf16 *>(p.cs_in) + (size_t)slot * 3 * CCH : nullptr;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        x[i] = csn ? *reinterpret_cast<const uint32_t *>(csn + (size_t)i * CCH + ch) : 0u;
}

__device__ __forceinline__ void load_early(const SplitParams &p, const SubTask &tk, int h, int lane, EarlyRows &r) {
    constexpr int D = kHeadDim;
    typedef __bf16 T;
    const int64_t rowbytes = (int64_t)p.H * D * 2;
    const RowWindow wa = row_window(tk, 0), wk = row_window(tk, -3);
    const __amdgpu_buffer_rsrc_t ra = row_rsrc(p.gate, tk, h, wa, rowbytes);
    const __amdgpu_buffer_rsrc_t rk = row_rsrc(p.k, tk, h, wk, rowbytes);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
        r.xa[rr] = __builtin_amdgcn_raw_buffer_load_b32(ra, 4 * lane, row_soff(wa, rr, rowbytes), 0);
#pragma unroll
    for (int i = 0; i < 19; ++i)
        r.xk[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane, row_soff(wk, i - 3, rowbytes), 0);
    // unconditional load from a row inside the sequence; the conversion and the
    // mask wait for the use, so this load does not force a wait on the others
    int br = 16 * (int)tk.j + (lane & 15);
    br = br < (int)tk.L ? br : (int)tk.L - 1;
    r.beta_bits = *reinterpret_cast<const unsigned short *>(reinterpret_cast<const T *>(p.beta) + (tk.s0 + br) * p.H + h);
    if (tk.j == 0) load_history(p, tk, h, lane, 1, r.xk);
}

__device__ __forceinline__ void load_late(const SplitParams &p, const SubTask &tk, int h, int lane, LateRows &r) {
    constexpr int D = kHeadDim;
    const int64_t rowbytes = (int64_t)p.H * D * 2;
    const RowWindow wr = row_window(tk, -3);
    const __amdgpu_buffer_rsrc_t rq = row_rsrc(p.q, tk, h, wr, rowbytes);
    const __amdgpu_buffer_rsrc_t rv = row_rsrc(p.v, tk, h, wr, rowbytes);
#pragma unroll
    for (int i = 0; i < 19; ++i) {
        const int so = row_soff(wr, i - 3, rowbytes);
        r.xq[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, so, 0);
        r.xv[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, 4 * lane, so, 0);
    }
    if (tk.j == 0) {
        load_history(p, tk, h, lane, 0, r.xq);
        load_history(p, tk, h, lane, 2, r.xv);
    }
}

// One 16-token sub-chunk by one wave, from its early and late rows (loads
// issued before).  When nx is set it starts the loads of the next sub-chunk's
// rows as soon as their registers are free: the early rows after the k block
// (into ner), the late rows after the v conv (into lr), so that they land while
// this sub-chunk finishes.  All LDS traffic stays inside the wave's region.
__device__ __forceinline__ void intra_sub_chunk(const SplitParams &p, unsigned char *lds, const SubTask &tk,
                                                int h, int lane, const EarlyRows &er, LateRows &lr,
                                                const ConvW &cw, const SubTask *nx, EarlyRows &ner) {
    constexpr int D = kHeadDim;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int64_t s0 = tk.s0, L = tk.L, j = tk.j;
    const int64_t p0 = 16 * j;
    const int rem = (int)(L - p0);  // rows of the sequence from p0 on (32-bit: scalar compares)
    const bool edge = p0 < 3 || rem < 16;
    const bool silu = p.flags & KDA_F_SILU;
    const bool l2 = !(p.flags & KDA_F_NO_QK_L2NORM);
    const bool glog = p.flags & KDA_F_GATE_IS_LOG;
    const int c0 = 2 * lane;
    __bf16 *sKL = reinterpret_cast<__bf16 *>(lds + A_KL);
    __bf16 *sQL = reinterpret_cast<__bf16 *>(lds + A_QL);
    __bf16 *sKI = reinterpret_cast<__bf16 *>(lds + A_KI);
    __bf16 *sKGT = reinterpret_cast<__bf16 *>(lds + A_KGT);
    __bf16 *sVT = reinterpret_cast<__bf16 *>(lds + A_VT);
    __bf16 *sPS = reinterpret_cast<__bf16 *>(lds + A_PS);
    unsigned char *rec = p.ws + ((size_t)h * p.nslots + tk.slot) * kRec;
    const uint32_t(&xq)[19] = lr.xq;
    const uint32_t(&xk)[19] = er.xk;
    const uint32_t(&xv)[19] = lr.xv;
    const uint32_t(&xa)[16] = er.xa;
    const float beta_r = (lane < 16 && lane < rem) ? __uint_as_float(er.beta_bits << 16) : 0.f;
    auto load_w = [&](int t, float (&wt)[2][4], float (&bs)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
            for (int i = 0; i < 4; ++i) wt[e][i] = cw.w[t][e][i];
            bs[e] = cw.b[t][e];
        }
    };
    // activation and the rows past the sequence end (zero contribution)
    auto finish = [&](float (&y)[16][2]) {
        if (silu) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                for (int e = 0; e < 2; ++e) y[rr][e] *= sigmoidf_dev(y[rr][e]);
        }
        if (edge) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                if (rr >= rem) { y[rr][0] = 0.f; y[rr][1] = 0.f; }
        }
    };
    float bt[16];  // beta per row, wave-uniform
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
        bt[rr] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(beta_r), rr));

    // ---- gate: log2 decays as running products from the sub-chunk start
    //   run_r = 2^{b_r},  back_r = 2^{b_last - b_r},  fd = 2^{-b_last}
    float run[16][2], back[16][2], fd[2];
    float g2v[2][16];
    if (glog) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) g2v[e][rr] = fmaxf(bf_ch(xa[rr], e), p.lb) * kLog2eS;
    } else {
        const float c = p.lb * kLog2eS;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) g2v[e][rr] = c * sigmoidf_dev(bf_ch(xa[rr], e));
    }
    if (edge) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            if (rr >= rem) g2v[0][rr] = g2v[1][rr] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        float al[16], r = 1.f, gs = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float g2 = g2v[e][rr];
            al[rr] = exp2_fast(g2);
            gs += g2;
            r *= al[rr];
            run[rr][e] = r;
        }
        float bk = 1.f;
#pragma unroll
        for (int rr = 15; rr >= 0; --rr) {
            back[rr][e] = bk;
            bk *= al[rr];
        }
        fd[e] = exp2_fast(-gs);
        run[15][e] = exp2_fast(gs);  // equal up to rounding; the record takes the direct form
    }
    {
        f32x2 gm = {run[15][0], run[15][1]};
        *reinterpret_cast<f32x2 *>(rec + R_GAM + 4 * c0) = gm;
    }

    // ---- k: KL = K.2^b, KI = K.2^-b (row-major), beta KL transposed, KD = K.2^(b_last-b)
    {
        float wt[2][4], bs[2], y[16][2], rk[16];
        load_w(1, wt, bs);
        conv16(xk, wt, bs, y);
        finish(y);
        l2_scale(y, l2, lane, rk);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            float kl[4][2], kr[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q4 + i;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float kn = y[r][e] * rk[r];
                    kl[i][e] = kn * run[r][e];
                    kr[i][e] = kn * back[r][e];
                }
                Pair<__bf16>::store(sKL + r * A_SRM + c0, kl[i][0], kl[i][1]);
                Pair<__bf16>::store(sKI + r * A_SRM + c0, kr[i][0] * fd[0], kr[i][1] * fd[1]);
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = c0 + e, r = 4 * q4;
                OPB::store4(sKGT + c * A_STR + r, bt[r] * kl[0][e], bt[r + 1] * kl[1][e],
                            bt[r + 2] * kl[2][e], bt[r + 3] * kl[3][e]);
                // accumulator / A-fragment layouts for pass B: element (token r, channel c)
                // of tile c / 16 sits in lane (r / 4) * 16 + c % 16, slot r % 4
                const size_t fo = ((size_t)((c >> 4) * 64 + q4 * 16 + (c & 15)) * 4) * 2;
                OPB::store4(reinterpret_cast<__bf16 *>(rec + R_KD + fo), kr[0][e], kr[1][e],
                            kr[2][e], kr[3][e]);
            }
        }
    }
    if (nx) load_early(p, *nx, h, lane, ner);
    // ---- q: QL = Q.2^b (row-major)
    {
        float wt[2][4], bs[2], y[16][2], rq[16];
        load_w(0, wt, bs);
        conv16(xq, wt, bs, y);
        finish(y);
        l2_scale(y, l2, lane, rq);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            Pair<__bf16>::store(sQL + rr * A_SRM + c0, y[rr][0] * rq[rr] * run[rr][0],
                                y[rr][1] * rq[rr] * run[rr][1]);
    }
    wave_sync_lds();

    // ---- decayed Grams over the sub-chunk (one 16 x 16 tile each).  N = diag(beta)
    // strict_lower(A) stays in registers in accumulator layout (row 4 g4 + i,
    // column m16 in slot i) for the inverse; P goes to LDS for its transpose.
    float nacc[4];
    {
        const f32x4 a = OPB::gram(sKL + m16 * A_SRM, sKI + m16 * A_SRM, nullptr, g4);
        const f32x4 pq = OPB::gram(sQL + m16 * A_SRM, sKI + m16 * A_SRM, nullptr, g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 4 * g4 + i, sl = m16;
            // beta of row rl (lanes 0..15 of beta_r hold rows 0..15), read as scalars and selected
            const int bb = __float_as_int(beta_r);
            const float b0 = __int_as_float(__builtin_amdgcn_readlane(bb, i));
            const float b1 = __int_as_float(__builtin_amdgcn_readlane(bb, 4 + i));
            const float b2 = __int_as_float(__builtin_amdgcn_readlane(bb, 8 + i));
            const float b3 = __int_as_float(__builtin_amdgcn_readlane(bb, 12 + i));
            const float brl = g4 < 2 ? (g4 == 0 ? b0 : b1) : (g4 == 2 ? b2 : b3);
            nacc[i] = (sl < rl) ? a[i] * brl : 0.f;
            sPS[rl * A_STR + sl] = (__bf16)((sl <= rl) ? pq[i] : 0.f);
        }
    }
    // Q . 2^b fragments (pairs of 16-channel blocks, matching pass B's state tiles)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const __bf16 *row = sQL + m16 * A_SRM + 32 * t + 4 * g4;
        bf16x8 f = join8(*reinterpret_cast<const bf16x4 *>(row), *reinterpret_cast<const bf16x4 *>(row + 16));
        *reinterpret_cast<bf16x8 *>(rec + R_QG + ((size_t)t * 64 + lane) * 16) = f;
    }
    wave_sync_lds();
    *reinterpret_cast<bf16x4 *>(rec + R_PP + (size_t)lane * 8) =
        *reinterpret_cast<const bf16x4 *>(sPS + m16 * A_STR + 4 * g4);

    // ---- v: beta V transposed into the dead QL area
    {
        float wt[2][4], bs[2], y[16][2];
        load_w(2, wt, bs);
        conv16(xv, wt, bs, y);
        if (nx) load_late(p, *nx, h, lane, lr);
        finish(y);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int r = 4 * q4;
                OPB::store4(sVT + (c0 + e) * A_VTS + r, bt[r] * y[r][e], bt[r + 1] * y[r + 1][e],
                            bt[r + 2] * y[r + 2][e], bt[r + 3] * y[r + 3][e]);
            }
    }
    // ---- X = (I + N)^-1, one row per lane: lane r (mod 16) solves
    // x (I + N) = e_r from the last column down, x_c = [c == r] - sum_{s > c} x_s N[s][c],
    // with N[s][c] read as a wave-uniform scalar from the register tile.  The
    // term with x_{c+1} comes last, so the dependent chain is one FMA per column.
    bf16x4 xfr;  // row m16 of X, columns 4 g4 .. 4 g4 + 3 (A-operand fragment)
    {
        float x[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) x[c] = (c == m16) ? 1.f : 0.f;
#pragma unroll
        for (int c = 14; c >= 0; --c) {
            float acc = x[c];
#pragma unroll
            for (int s = 15; s > c; --s) {
                const float nsc = __int_as_float(
                    __builtin_amdgcn_readlane(__float_as_int(nacc[s & 3]), 16 * (s >> 2) + c));
                acc = fmaf(-nsc, x[s], acc);
            }
            x[c] = acc;
        }
        // arithmetic selection by lane group (a select chain over x would be
        // turned into an indexed array access)
        const float m0 = g4 == 0 ? 1.f : 0.f, m1 = g4 == 1 ? 1.f : 0.f;
        const float m2 = g4 == 2 ? 1.f : 0.f, m3 = g4 == 3 ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xfr[i] = (__bf16)fmaf(x[i], m0, fmaf(x[4 + i], m1, fmaf(x[8 + i], m2, x[12 + i] * m3)));
    }
    wave_sync_lds();

    // ---- W = X diag(beta) (K . 2^b), staged row-major (negated) in the dead KL
    // area; U0 = X diag(beta) V straight to the record in accumulator layout
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int col = 16 * nt + m16;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 wr = mma_k16(xfr, OPB::load4raw(sKGT + col * A_STR + 4 * g4), z);
        const f32x4 ur = mma_k16(xfr, OPB::load4raw(sVT + col * A_VTS + 4 * g4), z);
#pragma unroll
        for (int i = 0; i < 4; ++i) sKL[(4 * g4 + i) * A_SRM + col] = (__bf16)(-wr[i]);
        *reinterpret_cast<bf16x4 *>(rec + R_U0 + ((size_t)nt * 64 + lane) * 8) = pack4(ur);
    }
    wave_sync_lds();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const __bf16 *row = sKL + m16 * A_SRM + 32 * t + 4 * g4;
        bf16x8 f = join8(*reinterpret_cast<const bf16x4 *>(row), *reinterpret_cast<const bf16x4 *>(row + 16));
        *reinterpret_cast<bf16x8 *>(rec + R_WN + ((size_t)t * 64 + lane) * 16) = f;
    }
}

// Pass A.  The slots of sequence n start at base(n) = start_n / 16 + n
// (strictly increasing in n); slot base(n) + j holds sub-chunk j of sequence n,
// and slots past the sequence's last sub-chunk are unused.  Wave w of the block
// for head h and slot group x takes slots x * 4 + w and x * 4 + w + 4 * (number
// of slot groups) of head h (the first valid ones from there), and loads the
// second one's rows while it computes the first.  Two slots in straight-line
// code: a loop over more slots keeps loop-invariant values live and spills.
__device__ __forceinline__ bool next_task(const SplitParams &p, int64_t slot, int64_t stride, SubTask &tk) {
    for (; slot < p.nslots; slot += stride) {
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            int64_t sm, lm;
            seq_bounds(p.cu, p.total, p.num_seqs, mid, sm, lm);
            if (sm / 16 + mid <= slot) lo = mid; else hi = mid - 1;
        }
        int64_t s0, L;
        seq_bounds(p.cu, p.total, p.num_seqs, lo, s0, L);
        const int64_t j = slot - (s0 / 16 + lo);
        if (16 * j < L) {
            tk.slot = slot; tk.s0 = s0; tk.L = L; tk.j = j; tk.n = lo;
            return true;
        }
    }
    return false;
}

__global__ void __launch_bounds__(256, 2) intra_kernel(SplitParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_a[];
    // the slot (and all derived from it) is wave-uniform: keep it scalar, so the
    // row buffer resources and offsets live in SGPRs
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // heads fastest when the grid allows, so that the workgroups resident at a
    // time read the same token rows of all heads together
    const int h = p.a_heads_fast ? blockIdx.x : blockIdx.y;
    const int64_t gb = p.a_heads_fast ? blockIdx.y : blockIdx.x;
    const int64_t stride = p.a_stride;
    unsigned char *lds = smem_a + w * A_WAVE;
    SubTask ta, tb;
    if (!next_task(p, gb * 4 + w, stride, ta)) return;
    ConvW cw;
    load_conv_w(p, h, lane, cw);
    EarlyRows ra, rb;
    LateRows lr;
    load_early(p, ta, h, lane, ra);
    load_late(p, ta, h, lane, lr);
    const bool hb = next_task(p, ta.slot + stride, stride, tb);
    intra_sub_chunk(p, lds, ta, h, lane, ra, lr, cw, hb ? &tb : nullptr, rb);
    if (hb) intra_sub_chunk(p, lds, tb, h, lane, rb, lr, cw, nullptr, ra);
}

// Pass B geometry.  Per 16-column dv tile one recurrence wave (R: all 128 dk
// rows of the state in registers) and one output wave (O), plus NP producer
// waves that fill an NS-stage LDS ring with the records by LDS DMA.  A stage
// holds a record's shared part and the NTW U0 tiles.  Per tile a double
// buffered exchange slot passes the bf16 S fragments and U from R to O.  The
// ring takes whatever LDS the exchange leaves (half of it at NTW = 1, where two
// workgroups share a CU), up to 10 stages.
template <int NTW> struct ScanGeom {
    static constexpr int kStage = R_U0 + NTW * 512;
    static constexpr int kInst = (kStage + 1023) / 1024;   // DMA instructions per stage
    static constexpr int NP = KDA_SCAN_PRODUCERS;          // producer waves
    // DMA instructions of producer pw per stage (it takes i = pw mod NP)
    static constexpr int inst_of(int pw) { return (kInst + NP - 1 - pw) / NP; }
    static constexpr int kInstP0 = inst_of(0);
    static constexpr int kWaves = 2 * NTW + NP;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kExSlot = 4096 + 512;             // S fragments + U fragment
    static constexpr int kExTile = 2 * kExSlot;
    static constexpr int kBudget = NTW == 1 ? 81920 : 163840;
    static constexpr int NSfit = (kBudget - NTW * kExTile) / kStage;
    static constexpr int NS = NSfit < 10 ? NSfit : 10;
    static constexpr int kExch = NS * kStage;              // exchange area offset
    static constexpr int kLds = kExch + NTW * kExTile;
    static constexpr int kMaxLater = NS - 3;
    static_assert(NS >= 4, "the ring holds the stages of steps j - 1, j, j + 1 and the refill");
    static_assert(kInstP0 * kMaxLater < 64, "in-flight DMA exceeds the vmcnt range");
    static_assert(NP >= 1 && NP <= 8 && kWaves <= 16 && kLds <= kBudget, "producers and LDS");
    static_assert(NTW == 1 || NTW == 2, "at most two dv tiles per workgroup");
};

// Lane K of each 16-lane row, broadcast to the whole row (DPP row_newbcast;
// every source lane exists, so bound_ctrl changes nothing but lets the
// compiler fold the move into the consuming multiply).
template <int K>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + K, 0xf, 0xf, true));
}

// s (dk tile M of the state, rows 16 M + 4 g4 + i) *= gam of those rows.  gv[q]
// holds, in lane (c, g4), gam of row 64 q + 16 (c >> 2) + 4 g4 + (c & 3), so the
// factor of row 16 M + 4 g4 + i sits in lane 4 (M & 3) + i of the same row.
template <int M>
__device__ __forceinline__ void decay_tile(f32x4 &s, const float (&gv)[2]) {
    s[0] *= row_bcast<4 * (M & 3) + 0>(gv[M >> 2]);
    s[1] *= row_bcast<4 * (M & 3) + 1>(gv[M >> 2]);
    s[2] *= row_bcast<4 * (M & 3) + 2>(gv[M >> 2]);
    s[3] *= row_bcast<4 * (M & 3) + 3>(gv[M >> 2]);
}

// Producer wait: everything but the DMA of the `later` most recently issued
// stages has landed (in-order completion of one wave's vector-memory ops).
template <int PER, int MAXL>
__device__ __forceinline__ void scan_wait(int later) {
    static_assert(MAXL <= 8 && PER * MAXL < 64, "cases below; the vmcnt range");
    // cases above MAXL are unreachable; their counts are clamped only to compile
    constexpr auto c = [](int k) { return PER * k < 64 ? PER * k : 63; };
    switch (later < MAXL ? later : MAXL) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<c(1)>(); break;
        case 2: wait_vmcnt<c(2)>(); break;
        case 3: wait_vmcnt<c(3)>(); break;
        case 4: wait_vmcnt<c(4)>(); break;
        case 5: wait_vmcnt<c(5)>(); break;
        case 6: wait_vmcnt<c(6)>(); break;
        case 7: wait_vmcnt<c(7)>(); break;
        default: wait_vmcnt<c(8)>(); break;
    }
}

// One producer wave with its index PW fixed at compile time, so that its share
// of a stage (instructions PW, PW + NP, ...) has constant offsets and its
// per-stage count PER is a constant.  Stages and record pointers advance
// incrementally; in the steady state the wait is a constant vmcnt, and the
// dispatch over the in-flight count runs only before B_-1 and in the tail.
template <int NTW, int PW>
__device__ __forceinline__ void producer_run(unsigned char *ring, const unsigned char *rec0, int nt0, int lane,
                                             int J) {
    typedef ScanGeom<NTW> G;
    constexpr int NS = G::NS, NP = G::NP, PER = G::inst_of(PW);
    auto issue = [&](int slot, const unsigned char *rec) {
        unsigned char *st = ring + slot * G::kStage;
#pragma unroll
        for (int i = PW; i < G::kInst; i += NP) {
            const int off = i * 1024 + lane * 16;  // byte within the stage
            if (off < G::kStage) {
                const unsigned char *src = off < R_U0 ? rec + off : rec + R_U0 + nt0 * 512 + (off - R_U0);
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(st + i * 1024), 16, 0, 0);
            }
        }
    };
    const int first = J < NS - 2 ? J : NS - 2;  // stages issued before B_-1
    const unsigned char *rec = rec0;
    for (int j = 0; j < first; ++j, rec += kRec) issue(j, rec);
    // B_-1 needs stage 0; stages 1 .. first - 1 may stay in flight
    scan_wait<PER, G::kMaxLater>(first - 1);
    __builtin_amdgcn_s_barrier();  // B_-1
    // steady state, b = 0 .. J - NS + 1: B_b needs stage b + 1 with NS - 4 later
    // stages in flight; after it, stage b + NS - 2 goes to slot (b + NS - 2) mod NS
    int slot = NS - 2;
    int b = 0;
    for (; b <= J - NS + 1; ++b, rec += kRec) {
        wait_vmcnt<PER * (NS - 4)>();
        __builtin_amdgcn_s_barrier();  // B_b
        issue(slot, rec);
        slot = slot + 1 == NS ? 0 : slot + 1;
    }
    // tail: nothing left to issue
    for (; b <= J; ++b) {
        if (b + 1 < J) scan_wait<PER, G::kMaxLater>(J - 1 - (b + 1));
        __builtin_amdgcn_s_barrier();  // B_b
    }
    wait_vmcnt<0>();
}

template <int NTW, int K = 0>
__device__ __forceinline__ void producer_dispatch(int pw, unsigned char *ring, const unsigned char *rec0, int nt0,
                                                  int lane, int J) {
    if constexpr (K < ScanGeom<NTW>::NP) {
        if (pw == K) {
            producer_run<NTW, K>(ring, rec0, nt0, lane, J);
            return;
        }
        producer_dispatch<NTW, K + 1>(pw, ring, rec0, nt0, lane, J);
    }
}

// Barriers, taken by every wave: B_-1, then B_j for j = 0 .. J.  At B_-1
// stage 0 is in LDS; at B_j stage j + 1 is (when j + 1 < J).  During step j
// the R waves compute from registers read from stage j and read stage j + 1;
// O reads stage j - 1 and the S and U fragments of step j - 1; after B_j the
// producers refill the slot of stage j - 2 with stage j + NS - 2.
template <int NTW>
__global__ void __launch_bounds__(ScanGeom<NTW>::kThreads, NTW == 1 ? 2 : 1) scan_kernel(SplitParams p) {
    typedef ScanGeom<NTW> G;
    constexpr int D = kHeadDim, NS = G::NS;
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
    // the wave index is uniform: keep it scalar so that role branches stay scalar
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int bid = blockIdx.x;
    const int grp = bid / (8 * p.tiles), rem = bid - grp * 8 * p.tiles;
    const int tile = rem >> 3, pr = grp * 8 + (rem & 7);
    if (pr >= p.pairs) return;  // whole workgroup: no barrier is left waiting
    const int H = p.H;
    const int n = pr / H, h = pr - n * H;
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup: no barrier is left waiting
    const size_t spr = (size_t)slot * H + h;  // pool row of this (sequence, head)
    int64_t s0, L;
    seq_bounds(p.cu, p.total, p.num_seqs, n, s0, L);
    const int64_t J = (L + 15) / 16;
    const int nt0 = tile * NTW;
    const unsigned char *rec0 =
        p.ws + ((size_t)h * p.nslots + (J > 0 ? sub_slot(s0, 0, n) : 0)) * kRec;
    auto stage = [&](int64_t j) { return ring + ((uint32_t)j % NS) * G::kStage; };

    if (w >= 2 * NTW) {
        // ---------------- producers
        // bare barriers throughout: a fence would drain all DMA in flight
        if (J == 0) return;
        producer_dispatch<NTW>(w - 2 * NTW, ring, rec0, nt0, lane, (int)J);
        return;
    }

    const bool is_r = w < NTW;
    const int tw = is_r ? w : w - NTW;  // tile within the workgroup
    const int nt = nt0 + tw;
    const int col = 16 * nt + m16;
    unsigned char *exch = ring + G::kExch + tw * G::kExTile;

    if (is_r) {
        // ---------------- recurrence on the 128 x 16 state block of tile nt:
        //   U = U0 - W S, S = diag(gam) S + Kd^T U
        // S[m] holds rows 16 m + 4 g4 + i of column col (accumulator layout).
        f32x4 S[8];
        if (p.state_in && p.state_bf16) {
            const __bf16 *sin = reinterpret_cast<const __bf16 *>(p.state_in) + spr * D * D + col;
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[m][i] = (float)sin[(16 * m + 4 * g4 + i) * D];
        } else if (p.state_in) {
            const float *sin = reinterpret_cast<const float *>(p.state_in) + spr * D * D + col;
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[m][i] = sin[(16 * m + 4 * g4 + i) * D];
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (J > 0) {
            int rslot = 1 % NS;  // ring slot of stage j + 1 during step j
            // A step's operands, read from the ring one step ahead: W (negated),
            // Kd, gam (one row per lane, see decay_tile) and this tile's U0.
            auto load = [&](const unsigned char *st, bf16x8 (&wn)[4], bf16x4 (&kd)[8], float (&gv)[2],
                            bf16x4 &u0) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    wn[t] = *reinterpret_cast<const bf16x8 *>(st + R_WN + (t * 64 + lane) * 16);
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    kd[m] = *reinterpret_cast<const bf16x4 *>(st + R_KD + (m * 64 + lane) * 8);
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    gv[q] = *reinterpret_cast<const float *>(
                        st + R_GAM + (64 * q + 16 * (m16 >> 2) + 4 * g4 + (m16 & 3)) * 4);
                u0 = *reinterpret_cast<const bf16x4 *>(st + R_U0 + (tw * 64 + lane) * 8);
            };
            // One step: operands of step j in the first set; the second set
            // receives step j + 1's (the loop alternates the two sets).
            auto step = [&](int64_t j, const bf16x8 (&wn)[4], const bf16x4 (&kd)[8], const float (&gv)[2],
                            bf16x4 u0, bf16x8 (&wn_n)[4], bf16x4 (&kd_n)[8], float (&gv_n)[2], bf16x4 &u0_n) {
                barrier_lds();  // B_j
                __builtin_amdgcn_sched_barrier(0);
                // (past the last step this reads a stale stage: harmless, and it keeps
                // the step one basic block so that the issue order below holds)
                load(ring + rslot * G::kStage, wn_n, kd_n, gv_n, u0_n);
                rslot = rslot + 1 == NS ? 0 : rslot + 1;
                bf16x8 Sp[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) Sp[t] = join8(pack4(S[2 * t]), pack4(S[2 * t + 1]));
                // two independent accumulation chains over the dk quarters
                f32x4 Ua = {(float)u0.x, (float)u0.y, (float)u0.z, (float)u0.w};
                f32x4 Uc = {0.f, 0.f, 0.f, 0.f};
                Ua = mma_k32(wn[0], Sp[0], Ua);
                Uc = mma_k32(wn[1], Sp[1], Uc);
                Ua = mma_k32(wn[2], Sp[2], Ua);
                Uc = mma_k32(wn[3], Sp[3], Uc);
                unsigned char *ex = exch + (j & 1) * G::kExSlot;
#pragma unroll
                for (int t = 0; t < 4; ++t) *reinterpret_cast<bf16x8 *>(ex + t * 1024 + lane * 16) = Sp[t];
                decay_tile<0>(S[0], gv);
                decay_tile<1>(S[1], gv);
                decay_tile<2>(S[2], gv);
                decay_tile<3>(S[3], gv);
                decay_tile<4>(S[4], gv);
                decay_tile<5>(S[5], gv);
                decay_tile<6>(S[6], gv);
                decay_tile<7>(S[7], gv);
                const bf16x4 Ub = pack4(Ua + Uc);
                *reinterpret_cast<bf16x4 *>(ex + 4096 + lane * 8) = Ub;
#pragma unroll
                for (int m = 0; m < 8; ++m) S[m] = mma_k16(kd[m], Ub, S[m]);
                // issue order: next operands; S_j to bf16 interleaved with the U
                // products; the decay under their latency; the S_j exchange; U; the
                // U exchange; the state products (the barrier's LDS wait then finds
                // the writes done)
                __builtin_amdgcn_sched_group_barrier(0x100, 11, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            };
            bf16x8 wnA[4], wnB[4];
            bf16x4 kdA[8], kdB[8], u0A, u0B = {};
            float gvA[2], gvB[2];
            barrier_lds();  // B_-1
            load(stage(0), wnA, kdA, gvA, u0A);
            int64_t j = 0;
            for (; j + 1 < J; j += 2) {
                step(j, wnA, kdA, gvA, u0A, wnB, kdB, gvB, u0B);
                step(j + 1, wnB, kdB, gvB, u0B, wnA, kdA, gvA, u0A);
            }
            if (j < J) step(j, wnA, kdA, gvA, u0A, wnB, kdB, gvB, u0B);
            barrier_lds();  // B_J
        }
        if (p.state_out) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t at = (spr * D + 16 * m + 4 * g4 + i) * D + col;
                    if (p.state_bf16)
                        reinterpret_cast<__bf16 *>(p.state_out)[at] = (__bf16)S[m][i];
                    else
                        reinterpret_cast<float *>(p.state_out)[at] = S[m][i];
                }
        }
        return;
    }

    // ---------------- output: O = scale ((Q . 2^b) S + P U) of step j - 1
    if (J == 0) return;
    const int64_t tokstride = (int64_t)H * D;
    // stores: a wave-uniform row base plus one 32-bit per-lane offset (column col
    // of row 4 g4 of the group), so the per-row address arithmetic is scalar
    __bf16 *ob = reinterpret_cast<__bf16 *>(p.o) + ((size_t)s0 * tokstride + (size_t)h * D);
    const uint32_t loff = (uint32_t)col + 4u * (uint32_t)g4 * (uint32_t)tokstride;
    int oslot = 0;  // ring slot of stage j - 1
    barrier_lds();  // B_-1
    for (int64_t j = 0; j <= J; ++j) {
        barrier_lds();  // B_j
        if (j > 0) {
            const int64_t jo = j - 1;
            const unsigned char *st = ring + oslot * G::kStage;
            oslot = oslot + 1 == NS ? 0 : oslot + 1;
            const unsigned char *ex = exch + (jo & 1) * G::kExSlot;
            // every operand first (one LDS round trip), then the product chain
            bf16x8 qg[4], sp[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                qg[t] = *reinterpret_cast<const bf16x8 *>(st + R_QG + (t * 64 + lane) * 16);
                sp[t] = *reinterpret_cast<const bf16x8 *>(ex + t * 1024 + lane * 16);
            }
            const bf16x4 pp = *reinterpret_cast<const bf16x4 *>(st + R_PP + lane * 8);
            const bf16x4 ub = *reinterpret_cast<const bf16x4 *>(ex + 4096 + lane * 8);
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) O = mma_k32(qg[t], sp[t], O);
            O = mma_k16w(pp, ub, O);  // the accumulator comes from K = 32 steps
            __bf16 *orow = ob + (size_t)(16 * jo) * tokstride;
            if (16 * jo + 16 <= L) {  // the whole sub-chunk lies in the sequence
#pragma unroll
                for (int i = 0; i < 4; ++i) (orow + (size_t)i * tokstride)[loff] = (__bf16)(p.scale * O[i]);
            } else {
                const int64_t r0 = 16 * jo + 4 * g4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (r0 + i < L) (orow + (size_t)i * tokstride)[loff] = (__bf16)(p.scale * O[i]);
            }
        }
    }
}

template <int NTW>
hipError_t launch_scan(const SplitParams &sp, hipStream_t s) {
    typedef ScanGeom<NTW> G;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_kernel<NTW>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    });
    if (attr != hipSuccess) return attr;
    const unsigned blocks = (unsigned)((sp.pairs + 7) / 8) * 8u * (unsigned)sp.tiles;
    hipLaunchKernelGGL(scan_kernel<NTW>, dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    return hipGetLastError();
}

}  // namespace

size_t split_workspace_bytes(int64_t total_tokens, int num_seqs, int H) {
    return (size_t)H * (size_t)(total_tokens / 16 + num_seqs) * kRec;
}

hipError_t launch_prefill_split(const kda_prefill_args *a, int dv_tile, hipStream_t s) {
    SplitParams sp;
    sp.q = a->q; sp.k = a->k; sp.v = a->v; sp.gate = a->gate; sp.beta = a->beta;
    sp.w = a->conv_weight; sp.bias = a->conv_bias; sp.cs_in = a->conv_state_in;
    sp.state_in = a->state_in; sp.state_out = a->state_out; sp.o = a->o;
    sp.state_bf16 = (a->flags & KDA_F_STATE_BF16) ? 1 : 0;
    sp.slots = a->state_slots; sp.num_slots = a->num_slots;
    sp.cu = a->cu_seqlens; sp.ws = static_cast<unsigned char *>(a->workspace);
    sp.total = a->total_tokens; sp.nslots = a->total_tokens / 16 + a->num_seqs;
    sp.num_seqs = a->num_seqs; sp.H = a->num_heads;
    sp.scale = a->scale; sp.lb = a->gate_lower_bound; sp.flags = a->flags;
    sp.pairs = a->num_seqs * a->num_heads;
    sp.a_heads_fast = 0;
    sp.a_stride = 0;
    if (dv_tile > 32) dv_tile = 32;  // at most two dv tiles of 16 columns per workgroup
    sp.tiles = kHeadDim / dv_tile;
    if (a->total_tokens > 0) {
        static std::once_flag once;
        static hipError_t attr = hipSuccess;
        std::call_once(once, [] {
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&intra_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 4 * A_WAVE);
        });
        if (attr != hipSuccess) return attr;
        // two slots per wave: wave (x, w) owns slots x * 4 + w + k * 4 * gx and takes
        // the valid ones, so 8 * gx must cover every valid slot index.  Those are
        // below ceil(total / 16) + num_seqs - 1 (the slot past a sequence's last
        // sub-chunk is never valid), which for one 16-aligned sequence is the
        // sub-chunk count itself and leaves no partly filled last round.
        const int64_t span = (a->total_tokens + 15) / 16 + a->num_seqs - 1;
        const int64_t gx = (span + 7) / 8;
        sp.a_heads_fast = gx <= 65535;
        sp.a_stride = 4 * gx;
        const dim3 grid = sp.a_heads_fast ? dim3((unsigned)a->num_heads, (unsigned)gx)
                                          : dim3((unsigned)gx, (unsigned)a->num_heads);
        hipLaunchKernelGGL(intra_kernel, grid, dim3(256), 4 * A_WAVE, s, sp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return dv_tile == 16 ? launch_scan<1>(sp, s) : launch_scan<2>(sp, s);
}

}  // namespace kda
