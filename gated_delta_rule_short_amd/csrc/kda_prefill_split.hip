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
//     X = (I + diag(beta) A)^-1,  W = X diag(beta) (K . 2^b),
// with b the log2-decay cumsum from the sub-chunk start (>= -115.4, so every
// factor is a finite fp32/bf16 number) and the output scale folded into the
// query side (Q~ = scale Q . 2^b), and writes them as matrix-core
// fragments to a workspace record, with X diag(beta) itself.  Pass B
// (scan_kernel) runs one workgroup per (sequence, head, dv tile) over its
// sub-chunks in order, forms U0 = X diag(beta) V from the conv of the raw v rows
// of its columns, and carries the state:
//     U = U0 - W S,  O = Q~ S + P U,
//     S = diag(2^b_last) S + (K . 2^(b_last - b))^T U.
// Pass A does the conv / L2 / gate work of q and k once per token and head,
// over the whole GPU; pass B keeps the fp32 state in registers (accumulator layout) for
// the whole sequence and streams the records through an LDS ring filled by
// producer waves with LDS DMA, so several sub-chunks are in flight while
// the consumer waves run the recurrence.  The workspace costs extra HBM
// traffic (one 13.5 KiB record per sub-chunk and head, written once and read
// once), which pays off when there are too few (sequence, head) pairs to fill
// the GPU otherwise.  v never enters the record: pass B reads its raw rows (the
// same bytes the record's V part would take) and pass A neither reads v nor
// writes U0.
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

// Record of one (head, sub-chunk), byte offsets; bf16 unless noted.
//   WN  [4][64][8]  -W, A-operand fragments (rows tokens, K = dk, permuted pairs)
//   QG  [4][64][8]  Q~ = scale Q . 2^b, same fragment layout
//   KD  [8][64][4]  (K . 2^(b_last - b))^T, A-operand fragments (rows dk, K = tokens)
//   PP  [64][4]     P, A-operand fragment (rows tokens, K = tokens)
//   GAM [128] fp32  2^b_last per dk channel
//   XB  [64][4]     X diag(beta), A-operand fragment (rows tokens, K = tokens)
// Every part is shared by all dv columns.  In LDS a record takes kRecArea bytes
// (whole DMA KiB; the tail past kRec receives duplicate bytes).  The fused
// schedule keeps its records in LDS only (kRec bytes a slot) and takes gam from a
// ring of its own.
constexpr int R_WN = 0, R_QG = 4096, R_KD = 8192, R_PP = 12288, R_GAM = 12800, R_XB = 13312;
constexpr size_t kRec = 13824;
constexpr int kRecArea = 14336;
constexpr int kRecInst = kRecArea / 1024;  // DMA instructions of a record
static_assert(kRecArea % 1024 == 0 && kRecArea >= (int)kRec && kRecArea - (int)kRec <= 512,
              "the last record DMA reads its tail twice");

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
    // Windows (jw > 0): the call runs in windows of jw sub-chunks of every sequence;
    // window `win` covers sub-chunks win * jw .. win * jw + jw - 1 of each sequence,
    // in slots n * jw + (j - win * jw), and the fp32 state of each (sequence, head)
    // waits in `carry` ([N][H][128][128]) from one window to the next.
    int64_t jw, win;
    float *carry;
    int spin_limit;  // polls of a fused hand-over wait before it gives up
};

// Slot of sub-chunk j of sequence n (start s0): distinct for all (n, j) and
// below total/16 + num_seqs, with consecutive j in consecutive slots.
__device__ __forceinline__ int64_t sub_slot(int64_t s0, int64_t j, int n) { return (s0 + 16 * j) / 16 + n; }

// Per-wave LDS of pass A (bytes).  Row-major tiles hold A_SRM bf16 per token
// row, transposed tiles A_STR bf16 per channel row.
constexpr int A_SRM = 132, A_STR = 20;
constexpr int A_KL = 0, A_QL = A_KL + 16 * A_SRM * 2, A_KI = A_QL + 16 * A_SRM * 2;
constexpr int A_KGT = A_KI + 16 * A_SRM * 2, A_PS = A_KGT + 128 * A_STR * 2;
constexpr int A_WAVE = A_PS + 16 * A_STR * 2;
static_assert(A_WAVE % 16 == 0, "wave region alignment");
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

// Per-row f / sqrt(sum of squares + eps) over the 128 channels (two per lane; a
// wave-uniform value per row), or f without the L2 step.
__device__ __forceinline__ void l2_scale(const float (&y)[16][2], bool l2, int lane, float f, float (&r)[16]) {
    if (!l2) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) r[rr] = f;
        return;
    }
    float p[16], s4[4];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) p[rr] = fmaf(y[rr][0], y[rr][0], y[rr][1] * y[rr][1]);
    rows16_sum(p, s4, lane);
#pragma unroll
    for (int t = 0; t < 4; ++t) s4[t] = __builtin_amdgcn_rsqf(s4[t] + 1e-6f) * f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) r[rr] = row_value(s4, rr);
}

// One pass-A task: sub-chunk j (rows 16 j .. 16 j + 15) of sequence n, which
// starts at token s0 and holds L tokens.
// Token positions are 32-bit (the token count is below 2^31), which keeps the
// per-row address arithmetic in single scalar instructions.
struct SubTask {
    int slot, s0, L, j, n;
};

// Raw inputs of one sub-chunk for this lane's two channels, as packed bf16
// pairs: rows p0-3 .. p0+15 of q and k (clamped into the sequence; the three
// rows before a sequence come from the conv state or are zero) and rows p0 ..
// p0+15 of the gate; beta of row p0 + lane in lanes 0..15.  The gate, k and
// beta ("early") are needed first and are loaded one sub-chunk ahead; q
// ("late") is loaded when the sub-chunk starts.
struct EarlyRows {
    uint32_t xk[19], xa[16];
    uint32_t beta_bits;  // raw bf16 of beta (row clamped into the sequence); masked at use
};
struct LateRows {
    uint32_t xq[19];
};

// Conv taps and bias of this lane's two q and k channels of head h.
struct ConvW {
    float w[2][2][4], b[2][2];
};

__device__ __forceinline__ void load_conv_w(const SplitParams &p, int h, int lane, ConvW &cw) {
    constexpr int D = kHeadDim;
    const int c0 = 2 * lane;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
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
    w.p0 = 16 * tk.j;
    w.L = tk.L;
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
// Byte offset of sub-chunk row r (-3 .. 15), clamped into the sequence, in the
// window: the rows lo .. hi are consecutive, so the clamp is one of the row index
// relative to lo into [0, hi - lo].
__device__ __forceinline__ int row_soff(const RowWindow &w, int r, int rowbytes) {
    int i = w.p0 - w.lo + r;
    i = i < 0 ? 0 : i;
    i = i > w.hi - w.lo ? w.hi - w.lo : i;
    return i * rowbytes;
}

// Every row p0 - 3 .. p0 + 15 of the task lies in its sequence: the row windows are
// exact and need no clamping.
__device__ __forceinline__ bool interior(const SubTask &tk) { return 16 * tk.j >= 3 && 16 * tk.j + 16 <= tk.L; }

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

// HIST = false: tk is known not to be the first sub-chunk of its sequence (no
// conv-state rows to fetch), which keeps the loads free of a conditional path.
template <bool HIST = true>
__device__ __forceinline__ void load_early(const SplitParams &p, const SubTask &tk, int h, int lane, EarlyRows &r) {
    constexpr int D = kHeadDim;
    typedef __bf16 T;
    const int64_t rowbytes = (int64_t)p.H * D * 2;
    const RowWindow wa = row_window(tk, 0), wk = row_window(tk, -3);
    const __amdgpu_buffer_rsrc_t ra = row_rsrc(p.gate, tk, h, wa, rowbytes);
    const __amdgpu_buffer_rsrc_t rk = row_rsrc(p.k, tk, h, wk, rowbytes);
    if (interior(tk)) {
        // no clamping: row i of a window at i rows from its start
        const int rb = (int)rowbytes;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) r.xa[rr] = __builtin_amdgcn_raw_buffer_load_b32(ra, 4 * lane, rr * rb, 0);
#pragma unroll
        for (int i = 0; i < 19; ++i) r.xk[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane, i * rb, 0);
    } else {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            r.xa[rr] = __builtin_amdgcn_raw_buffer_load_b32(ra, 4 * lane, row_soff(wa, rr, rowbytes), 0);
#pragma unroll
        for (int i = 0; i < 19; ++i)
            r.xk[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane, row_soff(wk, i - 3, rowbytes), 0);
    }
    // unconditional load from a row inside the sequence; the conversion and the
    // mask wait for the use, so this load does not force a wait on the others
    int br = 16 * tk.j + (lane & 15);
    br = br < tk.L ? br : tk.L - 1;
    r.beta_bits = *reinterpret_cast<const unsigned short *>(reinterpret_cast<const T *>(p.beta) +
                                                            ((size_t)tk.s0 + br) * p.H + h);
    if (HIST && tk.j == 0) load_history(p, tk, h, lane, 1, r.xk);
}

template <bool HIST = true>
__device__ __forceinline__ void load_late(const SplitParams &p, const SubTask &tk, int h, int lane, LateRows &r) {
    constexpr int D = kHeadDim;
    const int64_t rowbytes = (int64_t)p.H * D * 2;
    const RowWindow wr = row_window(tk, -3);
    const __amdgpu_buffer_rsrc_t rq = row_rsrc(p.q, tk, h, wr, rowbytes);
    if (interior(tk)) {
        const int rb = (int)rowbytes;
#pragma unroll
        for (int i = 0; i < 19; ++i) r.xq[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, i * rb, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 19; ++i)
            r.xq[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, row_soff(wr, i - 3, rowbytes), 0);
    }
    if (HIST && tk.j == 0) load_history(p, tk, h, lane, 0, r.xq);
}


// Lane K of each 16-lane row, broadcast to the whole row (DPP row_newbcast;
// every source lane exists, so bound_ctrl changes nothing but lets the
// compiler fold the move into the consuming multiply).
template <int K>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + K, 0xf, 0xf, true));
}

// Rows of X = (I + N)^-1 for a strictly lower 16 x 16 N, one row x per lane (x
// starts as the unit row e_r and comes out as row r of X): x_c = x_c + sum_{s > c}
// (-N[s][c]) x_s for every c.  Step k adds the term s = 15 - k to every column c <
// s at once; x_s is final by then (its last term came in step k - 1), and each
// column takes its terms in the order s = 15, 14, .., c + 1.  nneg[s] holds
// -N[s][c] in lane c of every 16-lane row, handed to the whole row by a DPP row
// broadcast inside v_fmac_f32 (the compiler does not fold a DPP move into a
// multiply-add, whose addend is tied to the result).  The FMAs of a step are
// independent, so the chain is 15 steps deep instead of 120.  Written out, the DPP
// read is invisible to the hazard check, so each step starts with the two wait
// states a DPP source needs after a VALU write of it.  The wave runs with every
// lane active here.
#define KDA_FMBC(c) "v_fmac_f32_dpp %[x" #c "], %[n], %[xs] row_newbcast:" #c " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void unit_lower_inverse_rows(float (&x)[16], const float (&nneg)[16]) {
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8) KDA_FMBC(9) KDA_FMBC(10) KDA_FMBC(11) KDA_FMBC(12) KDA_FMBC(13) KDA_FMBC(14)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), [x9] "+v"(x[9]), [x10] "+v"(x[10]), [x11] "+v"(x[11]), [x12] "+v"(x[12]), [x13] "+v"(x[13]), [x14] "+v"(x[14])
        : [n] "v"(nneg[15]), [xs] "v"(x[15]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8) KDA_FMBC(9) KDA_FMBC(10) KDA_FMBC(11) KDA_FMBC(12) KDA_FMBC(13)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), [x9] "+v"(x[9]), [x10] "+v"(x[10]), [x11] "+v"(x[11]), [x12] "+v"(x[12]), [x13] "+v"(x[13])
        : [n] "v"(nneg[14]), [xs] "v"(x[14]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8) KDA_FMBC(9) KDA_FMBC(10) KDA_FMBC(11) KDA_FMBC(12)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), [x9] "+v"(x[9]), [x10] "+v"(x[10]), [x11] "+v"(x[11]), [x12] "+v"(x[12])
        : [n] "v"(nneg[13]), [xs] "v"(x[13]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8) KDA_FMBC(9) KDA_FMBC(10) KDA_FMBC(11)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), [x9] "+v"(x[9]), [x10] "+v"(x[10]), [x11] "+v"(x[11])
        : [n] "v"(nneg[12]), [xs] "v"(x[12]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8) KDA_FMBC(9) KDA_FMBC(10)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), [x9] "+v"(x[9]), [x10] "+v"(x[10])
        : [n] "v"(nneg[11]), [xs] "v"(x[11]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8) KDA_FMBC(9)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), [x9] "+v"(x[9])
        : [n] "v"(nneg[10]), [xs] "v"(x[10]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7) KDA_FMBC(8)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8])
        : [n] "v"(nneg[9]), [xs] "v"(x[9]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6) KDA_FMBC(7)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7])
        : [n] "v"(nneg[8]), [xs] "v"(x[8]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5) KDA_FMBC(6)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6])
        : [n] "v"(nneg[7]), [xs] "v"(x[7]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4) KDA_FMBC(5)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5])
        : [n] "v"(nneg[6]), [xs] "v"(x[6]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3) KDA_FMBC(4)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4])
        : [n] "v"(nneg[5]), [xs] "v"(x[5]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2) KDA_FMBC(3)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3])
        : [n] "v"(nneg[4]), [xs] "v"(x[4]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1) KDA_FMBC(2)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2])
        : [n] "v"(nneg[3]), [xs] "v"(x[3]));
    asm("s_nop 1\n\t" KDA_FMBC(0) KDA_FMBC(1)
        : [x0] "+v"(x[0]), [x1] "+v"(x[1])
        : [n] "v"(nneg[2]), [xs] "v"(x[2]));
    asm("s_nop 1\n\t" KDA_FMBC(0)
        : [x0] "+v"(x[0])
        : [n] "v"(nneg[1]), [xs] "v"(x[1]));
}
#undef KDA_FMBC

// Conv taps and bias of one head in LDS (fused schedule): taps [3][128][4] for
// q, k, v, then biases [3][128]; fp32.
constexpr int kConvLdsBytes = 3 * 128 * 5 * 4;

// The head of one 16-token sub-chunk by one wave, from its early and late rows
// (loads issued before): the gate (gam into its ring entry), k (KD into the record
// at rec, KL, KI and KL transposed into the wave's tiles) and q (QL into its
// tile); brl receives beta of the lane's accumulator rows for the tail.  When nx is
// set it starts the loads of the next task's rows as soon as their registers are
// free: the early rows after the k block (into ner), the late rows after the last
// conv that reads them (into nlr).  All scratch LDS traffic stays inside the wave's
// region.  With LT (the fused schedule) the conv taps come from LDS (cwl) instead
// of registers (cw).  before_rec() runs right before the first write to rec (the
// fused schedule waits there for its ring slot, after the gate, which needs no
// slot).
template <bool LT, class BeforeRec>
__device__ __forceinline__ void intra_head(const SplitParams &p, unsigned char *lds, unsigned char *rec,
                                           const SubTask &tk, int h, int lane, const EarlyRows &er,
                                           const LateRows &lr, const ConvW &cw, const float *cwl,
                                           const SubTask *nx, EarlyRows &ner, LateRows &nlr,
                                           BeforeRec &&before_rec, float *gam, float (&brl)[4]) {
    constexpr int D = kHeadDim;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int p0 = 16 * tk.j;
    const int rem = tk.L - p0;  // rows of the sequence from p0 on
    const bool edge = p0 < 3 || rem < 16;
    const bool silu = p.flags & KDA_F_SILU;
    const bool l2 = !(p.flags & KDA_F_NO_QK_L2NORM);
    const bool glog = p.flags & KDA_F_GATE_IS_LOG;
    const int c0 = 2 * lane;
    __bf16 *sKL = reinterpret_cast<__bf16 *>(lds + A_KL);
    __bf16 *sQL = reinterpret_cast<__bf16 *>(lds + A_QL);
    __bf16 *sKI = reinterpret_cast<__bf16 *>(lds + A_KI);
    __bf16 *sKGT = reinterpret_cast<__bf16 *>(lds + A_KGT);
    __bf16 *sPS = reinterpret_cast<__bf16 *>(lds + A_PS);
    const uint32_t(&xq)[19] = lr.xq;
    const uint32_t(&xk)[19] = er.xk;
    const uint32_t(&xa)[16] = er.xa;
    const float beta_r = (lane < 16 && lane < rem) ? __uint_as_float(er.beta_bits << 16) : 0.f;
    auto load_w = [&](int t, float (&wt)[2][4], float (&bs)[2]) {
        if constexpr (LT) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(cwl + (t * 128 + c0 + e) * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) wt[e][i] = a[i];
            }
            const f32x2 b = *reinterpret_cast<const f32x2 *>(cwl + 3 * 128 * 4 + t * 128 + c0);
            bs[0] = b[0];
            bs[1] = b[1];
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wt[e][i] = cw.w[t][e][i];
                bs[e] = cw.b[t][e];
            }
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
    // beta of rows 4 g4 .. 4 g4 + 3 (the accumulator rows of this lane), from lanes
    // 4 g4 + i of beta_r
#pragma unroll
    for (int i = 0; i < 4; ++i)
        brl[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * g4 + i), __float_as_int(beta_r)));

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
        // c sigma(a) = 1 / ((1 + 2^(-a log2 e)) / c), the division by c folded into
        // one FMA with ic = 1 / c (kept finite, so that 2^(...) = 0 gives no 0 * inf)
        const float ic = fmaxf(1.f / (p.lb * kLog2eS), -3.0e38f);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const float ex = exp2_fast(-kLog2eS * bf_ch(xa[rr], e));
                g2v[e][rr] = __builtin_amdgcn_rcpf(fmaf(ex, ic, ic));
            }
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
    before_rec();
    {
        f32x2 gm = {run[15][0], run[15][1]};
        *reinterpret_cast<f32x2 *>(gam + c0) = gm;
    }

    // ---- k: KL = K.2^b, KI = K.2^-b (row-major), KL transposed, KD = K.2^(b_last-b)
    {
        float wt[2][4], bs[2], y[16][2], rk[16];
        load_w(1, wt, bs);
        conv16(xk, wt, bs, y);
        finish(y);
        l2_scale(y, l2, lane, 1.f, rk);
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
                OPB::store4(sKGT + c * A_STR + r, kl[0][e], kl[1][e], kl[2][e], kl[3][e]);
                // accumulator / A-fragment layouts for pass B: element (token r, channel c)
                // of tile c / 16 sits in lane (r / 4) * 16 + c % 16, slot r % 4
                const size_t fo = ((size_t)((c >> 4) * 64 + q4 * 16 + (c & 15)) * 4) * 2;
                OPB::store4(reinterpret_cast<__bf16 *>(rec + R_KD + fo), kr[0][e], kr[1][e],
                            kr[2][e], kr[3][e]);
            }
        }
    }
    // (only the two-pass schedule prefetches here; its next task may start a sequence)
    if (nx) load_early(p, *nx, h, lane, ner);
    // ---- q: QL = scale Q.2^b (row-major; the output scale rides on the query)
    {
        float wt[2][4], bs[2], y[16][2], rq[16];
        load_w(0, wt, bs);
        conv16(xq, wt, bs, y);
        if (nx) load_late(p, *nx, h, lane, nlr);
        finish(y);
        l2_scale(y, l2, lane, p.scale, rq);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            Pair<__bf16>::store(sQL + rr * A_SRM + c0, y[rr][0] * rq[rr] * run[rr][0],
                                y[rr][1] * rq[rr] * run[rr][1]);
    }
}

// The rest of a sub-chunk once its head has filled the wave's tiles (KL, KI, QL,
// KL transposed): the decayed Grams, the Q~ fragments and P, X diag(beta) and -W,
// into the record at rec.  brl: beta of the lane's accumulator rows, from the head.
__device__ __forceinline__ void intra_tail(unsigned char *lds, unsigned char *rec, int lane, const float (&brl)[4]) {
    const int m16 = lane & 15, g4 = lane >> 4;
    __bf16 *sKL = reinterpret_cast<__bf16 *>(lds + A_KL);
    __bf16 *sQL = reinterpret_cast<__bf16 *>(lds + A_QL);
    __bf16 *sKI = reinterpret_cast<__bf16 *>(lds + A_KI);
    __bf16 *sKGT = reinterpret_cast<__bf16 *>(lds + A_KGT);
    __bf16 *sPS = reinterpret_cast<__bf16 *>(lds + A_PS);
    wave_sync_lds();

    // ---- decayed Grams over the sub-chunk (one 16 x 16 tile each).  N = diag(beta)
    // strict_lower(A), negated, goes to LDS transposed (-N[s][c] at float 16 c + s,
    // in the K tile, which the Grams have finished with) for the inverse; P goes
    // to LDS for its transpose.
    float *sNT = reinterpret_cast<float *>(lds + A_KL);
    {
        const f32x4 a = OPB::gram(sKL + m16 * A_SRM, sKI + m16 * A_SRM, nullptr, g4);
        const f32x4 pq = OPB::gram(sQL + m16 * A_SRM, sKI + m16 * A_SRM, nullptr, g4);
        f32x4 nn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 4 * g4 + i, sl = m16;
            nn[i] = (sl < rl) ? -(a[i] * brl[i]) : 0.f;
            sPS[rl * A_STR + sl] = (__bf16)((sl <= rl) ? pq[i] : 0.f);
        }
        // rows 4 g4 .. 4 g4 + 3 of column m16 (the accumulator layout)
        *reinterpret_cast<f32x4 *>(sNT + 16 * m16 + 4 * g4) = nn;
    }
    // Q~ fragments (pairs of 16-channel blocks, matching pass B's state tiles)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const __bf16 *row = sQL + m16 * A_SRM + 32 * t + 4 * g4;
        bf16x8 f = join8(*reinterpret_cast<const bf16x4 *>(row), *reinterpret_cast<const bf16x4 *>(row + 16));
        *reinterpret_cast<bf16x8 *>(rec + R_QG + ((size_t)t * 64 + lane) * 16) = f;
    }
    wave_sync_lds();
    *reinterpret_cast<bf16x4 *>(rec + R_PP + (size_t)lane * 8) =
        *reinterpret_cast<const bf16x4 *>(sPS + m16 * A_STR + 4 * g4);

    // ---- X = (I + N)^-1, one row per lane: lane r (mod 16) solves
    // x (I + N) = e_r from the last column down, x_c = [c == r] - sum_{s > c} x_s N[s][c],
    // with -N[:, c] from LDS in lane c of every row, broadcast along the row.
    // row m16 of X diag(beta), columns 4 g4 .. 4 g4 + 3 (column 4 g4 + i carries beta of
    // row 4 g4 + i): the A-operand fragment of U0 = X diag(beta) V and the B operand
    // of W^T below
    bf16x4 xb;
    {
        float nneg[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sNT + 16 * m16 + 4 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) nneg[4 * q + i] = v[i];
        }
        float x[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) x[c] = (c == m16) ? 1.f : 0.f;
        unit_lower_inverse_rows(x, nneg);
        // arithmetic selection by lane group (a select chain over x would be
        // turned into an indexed array access)
        const float m0 = g4 == 0 ? 1.f : 0.f, m1 = g4 == 1 ? 1.f : 0.f;
        const float m2 = g4 == 2 ? 1.f : 0.f, m3 = g4 == 3 ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xb[i] = (__bf16)(fmaf(x[i], m0, fmaf(x[4 + i], m1, fmaf(x[8 + i], m2, x[12 + i] * m3))) * brl[i]);
        *reinterpret_cast<bf16x4 *>(rec + R_XB + (size_t)lane * 8) = xb;
    }
    wave_sync_lds();

    // ---- -W = -X diag(beta) (K . 2^b), formed transposed: -W^T = (K . 2^b)^T (-X diag(beta))^T
    // puts row r of W, channels 16 nt + 4 g4 .. + 3, in lane r + 16 g4 of tile nt,
    // which is the A-operand fragment pass B reads (tiles 2t and 2t + 1 give the two
    // halves of fragment t), so W goes to the record without an LDS round trip.  The
    // sign rides on the four bf16 of X diag(beta) (an exact sign flip), not on K.
    typedef uint32_t w2 __attribute__((ext_vector_type(2)));
    const bf16x4 xbn = __builtin_bit_cast(bf16x4, __builtin_bit_cast(w2, xb) ^ w2{0x80008000u, 0x80008000u});
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const f32x4 w0 = mma_k16(OPB::load4raw(sKGT + (32 * t + m16) * A_STR + 4 * g4), xbn, z);
        const f32x4 w1 = mma_k16(OPB::load4raw(sKGT + (32 * t + 16 + m16) * A_STR + 4 * g4), xbn, z);
        *reinterpret_cast<bf16x8 *>(rec + R_WN + ((size_t)t * 64 + lane) * 16) = join8(pack4(w0), pack4(w1));
    }
}

// One sub-chunk, head then tail (see intra_head and intra_tail).
template <bool LT, class BeforeRec>
__device__ __forceinline__ void intra_sub_chunk(const SplitParams &p, unsigned char *lds, unsigned char *rec,
                                                const SubTask &tk, int h, int lane, const EarlyRows &er,
                                                const LateRows &lr, const ConvW &cw, const float *cwl,
                                                const SubTask *nx, EarlyRows &ner, LateRows &nlr,
                                                BeforeRec &&before_rec, float *gam) {
    float brl[4];
    intra_head<LT>(p, lds, rec, tk, h, lane, er, lr, cw, cwl, nx, ner, nlr, before_rec, gam, brl);
    intra_tail(lds, rec, lane, brl);
}

// Pass A.  The slots of sequence n start at base(n) = start_n / 16 + n
// (strictly increasing in n); slot base(n) + j holds sub-chunk j of sequence n,
// and slots past the sequence's last sub-chunk are unused.  Wave w of the block
// for head h and slot group x takes slots x * 4 + w and x * 4 + w + 4 * (number
// of slot groups) of head h (the first valid ones from there), and loads the
// second one's rows while it computes the first.  Two slots in straight-line
// code: a loop over more slots keeps loop-invariant values live and spills.
__device__ __forceinline__ bool next_task(const SplitParams &p, int64_t slot, int64_t stride, SubTask &tk) {
    if (p.jw > 0) {  // windows: slot n * jw + i holds sub-chunk win * jw + i of sequence n
        for (; slot < p.nslots; slot += stride) {
            const int n = (int)(slot / p.jw);
            const int64_t j = p.win * p.jw + (slot - (int64_t)n * p.jw);
            int64_t s0, L;
            seq_bounds(p.cu, p.total, p.num_seqs, n, s0, L);
            if (16 * j < L) {
                tk.slot = slot; tk.s0 = s0; tk.L = L; tk.j = j; tk.n = n;
                return true;
            }
        }
        return false;
    }
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
    intra_sub_chunk<false>(p, lds, p.ws + ((size_t)h * p.nslots + ta.slot) * kRec, ta, h, lane, ra, lr, cw,
                           nullptr, hb ? &tb : nullptr, rb, lr, [] {},
                           reinterpret_cast<float *>(p.ws + ((size_t)h * p.nslots + ta.slot) * kRec + R_GAM));
    if (hb)
        intra_sub_chunk<false>(p, lds, p.ws + ((size_t)h * p.nslots + tb.slot) * kRec, tb, h, lane, rb, lr, cw,
                               nullptr, nullptr, ra, lr, [] {},
                               reinterpret_cast<float *>(p.ws + ((size_t)h * p.nslots + tb.slot) * kRec + R_GAM));
}

// Pass B geometry.  Per 16-column dv tile one recurrence wave (R: all 128 dk
// rows of the state in registers) and one output wave (O), plus NP producer
// waves that fill an NS-stage LDS ring by LDS DMA.  A stage holds a record and
// the 19 raw v rows (3 before the sub-chunk, 16 in it) of the workgroup's
// 16 NTW columns.  Per tile a double buffered exchange slot passes the bf16 S
// fragments and U from R to O, and O passes back U0 of the step after next,
// which it forms from the raw v rows (O issues no DMA, so its LDS reads never
// wait for the ring's copies).  The ring takes whatever
// LDS the exchange leaves (half of it at NTW = 1, where two workgroups share a
// CU), up to 10 stages.
template <int NTW> struct ScanGeom {
    static constexpr int kVRow = 32 * NTW;                      // bytes of a raw v row
    static constexpr int kVInst = (19 * kVRow + 1023) / 1024;   // DMA instructions of the v rows
    static constexpr int kVOff = kRecArea;                      // v rows within a stage
    static constexpr int kStage = kRecArea + kVInst * 1024;
    static constexpr int kInst = kRecInst + kVInst;             // DMA instructions per stage
    static constexpr int NP = KDA_SCAN_PRODUCERS;               // producer waves
    // DMA instructions of producer pw per stage (it takes i = pw mod NP)
    static constexpr int inst_of(int pw) { return (kInst + NP - 1 - pw) / NP; }
    static constexpr int kInstP0 = inst_of(0);
    // With two tiles a third wave per tile forms U0 (UW); one tile keeps it on the
    // recurrence wave, since seven waves would not leave two workgroups per CU
    // their registers.
    static constexpr bool UW = NTW == 2;
    static constexpr int kWaves = (UW ? 3 : 2) * NTW + NP;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kExSlot = 4096 + 512;             // S fragments + U fragment
    static constexpr int kU0Off = 2 * kExSlot;             // U0 of steps j, j + 1 (fp32), UW
    static constexpr int kExTile = 2 * kExSlot + (UW ? 2 * 1024 : 0);
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

// Raw v rows of a workgroup's columns for one sequence and head: `base` is the
// first column of the workgroup in row 0 of the sequence; rows are `rowbytes`
// apart; L is the sequence length.
struct VRows {
    const unsigned char *base;
    int64_t rowbytes;
    int L;
};

// Conv taps, bias and the three rows before the sequence (conv state, or zeros)
// of this lane's v column, for U0.
struct VConv {
    float w[4], b, hist[3];
};

__device__ __forceinline__ void load_vconv(const SplitParams &p, int slot, int h, int colh, bool first_window,
                                           VConv &vc) {
    constexpr int D = kHeadDim;
    const int ch = 2 * p.H * D + h * D + colh;  // v channel of the conv
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p.w + 4 * ch);
#pragma unroll
    for (int i = 0; i < 4; ++i) vc.w[i] = a[i];
    vc.b = p.bias ? p.bias[ch] : 0.f;
    const int CCH = 3 * p.H * D;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        vc.hist[i] = (first_window && p.cs_in)
                         ? (float)reinterpret_cast<const __bf16 *>(p.cs_in)[((size_t)slot * 3 + i) * CCH + ch]
                         : 0.f;
}

// U0 = X diag(beta) V of one 16-column tile from a stage: the width-4 conv of the
// raw v rows 4 g4 - 3 .. 4 g4 + 3 of the sub-chunk in this lane's column (byte
// colb of a row; at a sequence's first sub-chunk the three rows before it come
// from the conv state), SiLU with the flag, rounded to bf16, times the record's
// X diag(beta) fragment.  Rows past the sequence end hold clamped copies of its
// last row: finite, and X diag(beta) has zero columns for them.
template <int kVOff, int kVRow>
__device__ __forceinline__ f32x4 u0_tile(const unsigned char *st, int colb, int lane, bool first, const VConv &vc,
                                         bool silu) {
    const int g4 = lane >> 4;
    const unsigned char *vb = st + kVOff + colb + 4 * g4 * kVRow;
    float x[7];
#pragma unroll
    for (int r = 0; r < 7; ++r) x[r] = (float)*reinterpret_cast<const __bf16 *>(vb + r * kVRow);
    if (first && g4 == 0) {
        x[0] = vc.hist[0];
        x[1] = vc.hist[1];
        x[2] = vc.hist[2];
    }
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float a = fmaf(vc.w[0], x[i], vc.b);
        a = fmaf(vc.w[1], x[i + 1], a);
        a = fmaf(vc.w[2], x[i + 2], a);
        a = fmaf(vc.w[3], x[i + 3], a);
        y[i] = silu ? a * sigmoidf_dev(a) : a;
    }
    const bf16x4 xb = *reinterpret_cast<const bf16x4 *>(st + R_XB + lane * 8);
    // a K = 32 shape, as the U chain it starts
    return mma_k16w(xb, pack4(y), f32x4{0.f, 0.f, 0.f, 0.f});
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
template <class G, int PW>
__device__ __forceinline__ void producer_run(unsigned char *ring, const unsigned char *rec0, const VRows &vr,
                                             int64_t j0, int lane, int J) {
    constexpr int NS = G::NS, NP = G::NP, PER = G::inst_of(PW);
    // stage of sub-chunk jabs: the record (its last DMA reads the record's tail
    // twice, so every lane stays inside it) and the raw v rows 16 jabs - 3 ..
    // 16 jabs + 15 clamped into the sequence (lanes past row 18 repeat it).  Every
    // instruction is issued by every lane: PER per stage, exactly.
    auto issue = [&](int slot, const unsigned char *rec, int64_t jabs) {
        unsigned char *st = ring + slot * G::kStage;
#pragma unroll
        for (int i = PW; i < G::kInst; i += NP) {
            if (i < kRecInst) {
                const int off = i * 1024 + lane * 16;
                const int so = off < (int)kRec ? off : off - 512;
                __builtin_amdgcn_global_load_lds(rec + so, (lds_void *)(st + i * 1024), 16, 0, 0);
            } else {
                const int vi = i - kRecInst;
                const int byte = vi * 1024 + lane * 16;
                int r = byte / G::kVRow;
                const int cb = byte - r * G::kVRow;
                r = r > 18 ? 18 : r;
                int t = 16 * (int)jabs - 3 + r;
                t = t < 0 ? 0 : (t >= vr.L ? vr.L - 1 : t);
                __builtin_amdgcn_global_load_lds(vr.base + (size_t)t * vr.rowbytes + cb,
                                                 (lds_void *)(st + G::kVOff + vi * 1024), 16, 0, 0);
            }
        }
    };
    const int first = J < NS - 2 ? J : NS - 2;  // stages issued before B_-1
    const unsigned char *rec = rec0;
    int64_t jabs = j0;
    for (int j = 0; j < first; ++j, rec += kRec, ++jabs) issue(j, rec, jabs);
    // B_-1 needs stage 0; stages 1 .. first - 1 may stay in flight
    scan_wait<PER, G::kMaxLater>(first - 1);
    __builtin_amdgcn_s_barrier();  // B_-1
    // steady state, b = 0 .. J - NS + 1: B_b needs stage b + 1 with NS - 4 later
    // stages in flight; after it, stage b + NS - 2 goes to slot (b + NS - 2) mod NS
    int slot = NS - 2;
    int b = 0;
    for (; b <= J - NS + 1; ++b, rec += kRec, ++jabs) {
        wait_vmcnt<PER * (NS - 4)>();
        __builtin_amdgcn_s_barrier();  // B_b
        issue(slot, rec, jabs);
        slot = slot + 1 == NS ? 0 : slot + 1;
    }
    // tail: nothing left to issue
    for (; b <= J; ++b) {
        if (b + 1 < J) scan_wait<PER, G::kMaxLater>(J - 1 - (b + 1));
        __builtin_amdgcn_s_barrier();  // B_b
    }
    wait_vmcnt<0>();
}

template <class G, int K = 0>
__device__ __forceinline__ void producer_dispatch(int pw, unsigned char *ring, const unsigned char *rec0,
                                                  const VRows &vr, int64_t j0, int lane, int J) {
    if constexpr (K < G::NP) {
        if (pw == K) {
            producer_run<G, K>(ring, rec0, vr, j0, lane, J);
            return;
        }
        producer_dispatch<G, K + 1>(pw, ring, rec0, vr, j0, lane, J);
    }
}

// What one pass-B workgroup does in this call for sequence n, head h (pool row
// slot): its steps (sub-chunks j0 .. j0 + steps - 1), where its state comes from
// and goes to, and its first record.  Without windows that is the whole
// sequence, from state_in (or zeros) to state_out.  With windows, window 0 starts
// from state_in, later ones from the carry, and a window that does not hold the
// sequence's last sub-chunk leaves the state in the carry.  Returns false when the
// sequence has nothing in this window (an empty sequence passes its state through
// in window 0); the caller's whole workgroup then exits before any barrier.
struct PairWork {
    int64_t s0, L, j0, steps;
    const void *sin;
    void *sout;
    size_t sin_row, sout_row;
    bool sin16, sout16;
    const unsigned char *rec0;
};
// Sequence of rank r when the sequences are ordered by length, longest first (ties
// by index).  A pass-B or fused workgroup for (rank r, head) takes that sequence,
// so the longest sequences start first and the short ones fill in at the end,
// which shortens the tail of a launch whose workgroups run for very different
// times.  Every thread of the workgroup calls this with the same arguments; lens
// is LDS for kOrderMax + 1 ints.  The ranks of the N sequences are a permutation
// of 0 .. N - 1, so exactly one thread writes the result.  Without cu_seqlens
// (equal lengths) or with more than kOrderMax sequences the order is the index.
constexpr int kOrderMax = 256;
__device__ __forceinline__ bool order_by_length(const SplitParams &p) {
    return p.cu && p.num_seqs > 1 && p.num_seqs <= kOrderMax;
}
template <int kThreads>
__device__ __forceinline__ int seq_of_rank(const int32_t *cu, int N, int r, int *lens) {
    for (int i = threadIdx.x; i < N; i += kThreads) lens[i] = cu[i + 1] - cu[i];
    __syncthreads();
    for (int t = threadIdx.x; t < N; t += kThreads) {
        const int lt = lens[t];
        int rank = 0;
        for (int m = 0; m < N; ++m) {
            const int lm = lens[m];
            rank += (lm > lt || (lm == lt && m < t)) ? 1 : 0;
        }
        if (rank == r) lens[kOrderMax] = t;
    }
    __syncthreads();
    return lens[kOrderMax];
}

__device__ __forceinline__ bool pair_work(const SplitParams &p, int n, int h, int slot, PairWork &w) {
    seq_bounds(p.cu, p.total, p.num_seqs, n, w.s0, w.L);
    const int64_t J = (w.L + 15) / 16;
    const size_t spr = (size_t)slot * p.H + h;
    w.sin = p.state_in;
    w.sout = p.state_out;
    w.sin_row = w.sout_row = spr;
    w.sin16 = w.sout16 = p.state_bf16 != 0;
    w.j0 = 0;
    w.steps = J;
    int64_t first = J > 0 ? sub_slot(w.s0, 0, n) : 0;
    if (p.jw > 0) {
        w.j0 = p.win * p.jw;
        if (w.j0 >= J && !(p.win == 0 && J == 0)) return false;
        const int64_t j1 = J < w.j0 + p.jw ? J : w.j0 + p.jw;
        w.steps = j1 > w.j0 ? j1 - w.j0 : 0;
        const size_t crow = (size_t)n * p.H + h;
        if (p.win > 0) {
            w.sin = p.carry;
            w.sin_row = crow;
            w.sin16 = false;
        }
        if (j1 < J) {
            w.sout = p.carry;
            w.sout_row = crow;
            w.sout16 = false;
        }
        first = (int64_t)n * p.jw;
    }
    w.rec0 = p.ws + ((size_t)h * p.nslots + first) * kRec;
    return true;
}

// Rows 16 m + 4 g4 + i of state column col, accumulator layout, from or to state
// row `row` (fp32, or bf16 widened exactly / rounded to nearest even); a null
// source gives zeros, a null destination is not written.
__device__ __forceinline__ void load_state_tile(f32x4 (&S)[8], const void *src, size_t row, bool bf16, int col,
                                                int g4) {
    constexpr int D = kHeadDim;
    if (src && bf16) {
        const __bf16 *sin = reinterpret_cast<const __bf16 *>(src) + row * D * D + col;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[m][i] = (float)sin[(16 * m + 4 * g4 + i) * D];
    } else if (src) {
        const float *sin = reinterpret_cast<const float *>(src) + row * D * D + col;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[m][i] = sin[(16 * m + 4 * g4 + i) * D];
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}
__device__ __forceinline__ void store_state_tile(const f32x4 (&S)[8], void *dst, size_t row, bool bf16, int col,
                                                 int g4) {
    constexpr int D = kHeadDim;
    if (!dst) return;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t at = (row * D + 16 * m + 4 * g4 + i) * D + col;
            if (bf16)
                reinterpret_cast<__bf16 *>(dst)[at] = (__bf16)S[m][i];
            else
                reinterpret_cast<float *>(dst)[at] = S[m][i];
        }
}

// Barriers, taken by every wave: B_-1, then B_j for j = 0 .. J.  At B_-1
// stage 0 is in LDS; at B_j stage j + 1 is (when j + 1 < J).  During step j
// the R waves compute from registers read from stage j and read stage j + 1;
// O reads stage j - 1 and the S and U fragments of step j - 1; after B_j the
// producers refill the slot of stage j - 2 with stage j + NS - 2.
// SILU (KDA_F_SILU) is a template argument of the kernels that run the recurrence
// (this one, scan_wide_kernel and fused_kernel): with a run-time flag the compiler
// evaluates the activation of U0's conv in every step and selects the result
// afterwards.
template <int NTW, bool SILU>
__global__ void __launch_bounds__(ScanGeom<NTW>::kThreads, NTW == 1 ? 2 : 1) scan_kernel(SplitParams p) {
    typedef ScanGeom<NTW> G;
    constexpr int D = kHeadDim, NS = G::NS;
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
    // the wave index is uniform: keep it scalar so that role branches stay scalar.
    // Roles by index: recurrence waves, output waves, U0 waves, producers.  With two
    // tiles the U0 waves take hardware waves 6 and 7 and the first two producers
    // waves 4 and 5, so that a U0 wave shares its SIMD with an output wave rather
    // than with the MFMA-heavy recurrence wave (waves go round the four SIMDs).
    const int wh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int w = (NTW == 2 && wh >= 4 && wh < 8) ? (wh ^ 2) : wh;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int bid = blockIdx.x;
    const int grp = bid / (8 * p.tiles), rem = bid - grp * 8 * p.tiles;
    const int tile = rem >> 3, pr = grp * 8 + (rem & 7);
    if (pr >= p.pairs) return;  // whole workgroup: no barrier is left waiting
    const int H = p.H;
    const int rk = pr / H, h = pr - rk * H;
    int n = rk;
    if (order_by_length(p)) {
        // the ring's first bytes as scratch, before any wave writes the ring
        n = seq_of_rank<G::kThreads>(p.cu, p.num_seqs, rk, reinterpret_cast<int *>(ring));
        __syncthreads();
    }
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup: no barrier is left waiting
    PairWork pw;
    if (!pair_work(p, n, h, slot, pw)) return;  // whole workgroup: no barrier is left waiting
    const int64_t s0 = pw.s0, L = pw.L, j0 = pw.j0, J = pw.steps;
    const int nt0 = tile * NTW;
    const unsigned char *rec0 = pw.rec0;
    auto stage = [&](int64_t j) { return ring + ((uint32_t)j % NS) * G::kStage; };

    constexpr int kRole = G::UW ? 3 : 2;  // waves per tile
    if (w >= kRole * NTW) {
        // ---------------- producers
        // bare barriers throughout: a fence would drain all DMA in flight
        if (J == 0) return;
        const VRows vr{reinterpret_cast<const unsigned char *>(p.v) + ((size_t)s0 * H + h) * D * 2 + nt0 * 32,
                       (int64_t)H * D * 2, (int)L};
        producer_dispatch<G>(w - kRole * NTW, ring, rec0, vr, j0, lane, (int)J);
        return;
    }

    const bool is_r = w < NTW;
    const int tw = w % NTW;  // tile within the workgroup
    const int nt = nt0 + tw;
    const int col = 16 * nt + m16;
    unsigned char *exch = ring + G::kExch + tw * G::kExTile;

    if (G::UW && w >= 2 * NTW) {
        // ---------------- U0 of step j + 1 during step j (stage j + 1 is in LDS at
        // B_j), into the exchange slot of its step's parity
        if (J == 0) return;
        constexpr bool silu = SILU;
        VConv vc;
        load_vconv(p, slot, h, col, j0 == 0, vc);
        auto put_u0 = [&](int64_t js) {
            const f32x4 u0 = u0_tile<G::kVOff, G::kVRow>(stage(js), (tw * 16 + m16) * 2, lane, j0 + js == 0, vc,
                                                         silu);
            *reinterpret_cast<f32x4 *>(exch + G::kU0Off + (js & 1) * 1024 + lane * 16) = u0;
        };
        barrier_lds();  // B_-1
        put_u0(0);
        for (int64_t j = 0; j <= J; ++j) {
            barrier_lds();  // B_j
            if (j + 1 < J) put_u0(j + 1);
        }
        return;
    }

    if (is_r) {
        // ---------------- recurrence on the 128 x 16 state block of tile nt:
        //   U = U0 - W S, S = diag(gam) S + Kd^T U
        // S[m] holds rows 16 m + 4 g4 + i of column col (accumulator layout).
        f32x4 S[8];
        load_state_tile(S, pw.sin, pw.sin_row, pw.sin16, col, g4);
        if (J > 0) {
            int rslot = 1 % NS;  // ring slot of stage j + 1 during step j
            constexpr bool silu = SILU;
            VConv vc;
            if (!G::UW) load_vconv(p, slot, h, col, j0 == 0, vc);
            // A step's operands, read from the ring one step ahead: W (negated),
            // Kd, gam (one row per lane, see decay_tile) and, without a U0 wave,
            // U0 (formed from the raw v rows of the stage).
            auto load = [&](const unsigned char *st, int64_t jabs, bf16x8 (&wn)[4], bf16x4 (&kd)[8], f32x4 &u0,
                            float (&gv)[2]) {
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
                if (!G::UW) u0 = u0_tile<G::kVOff, G::kVRow>(st, (tw * 16 + m16) * 2, lane, jabs == 0, vc, silu);
            };
            // One step: operands of step j in the first set; the second set
            // receives step j + 1's (the loop alternates the two sets).
            auto step = [&](int64_t j, const bf16x8 (&wn)[4], const bf16x4 (&kd)[8], const f32x4 &u0,
                            const float (&gv)[2], bf16x8 (&wn_n)[4], bf16x4 (&kd_n)[8], f32x4 &u0_n,
                            float (&gv_n)[2]) {
                barrier_lds();  // B_j
                __builtin_amdgcn_sched_barrier(0);
                // with a U0 wave: this step's U0 from its exchange slot, added after
                // the products so that the read hides under them
                f32x4 u0w = {0.f, 0.f, 0.f, 0.f};
                if (G::UW) u0w = *reinterpret_cast<const f32x4 *>(exch + G::kU0Off + (j & 1) * 1024 + lane * 16);
                // (past the last step this reads a stale stage: harmless)
                load(ring + rslot * G::kStage, j0 + j + 1, wn_n, kd_n, u0_n, gv_n);
                rslot = rslot + 1 == NS ? 0 : rslot + 1;
                bf16x8 Sp[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) Sp[t] = join8(pack4(S[2 * t]), pack4(S[2 * t + 1]));
                // two independent accumulation chains over the dk quarters
                f32x4 Ua = G::UW ? f32x4{0.f, 0.f, 0.f, 0.f} : u0;
                f32x4 Uc = {0.f, 0.f, 0.f, 0.f};
                Ua = mma_k32(wn[0], Sp[0], Ua);
                Uc = mma_k32(wn[1], Sp[1], Uc);
                Ua = mma_k32(wn[2], Sp[2], Ua);
                Uc = mma_k32(wn[3], Sp[3], Uc);
                // The decays run while the U products are in flight: left to the
                // scheduler, most of them sat between U's pack and the state
                // products, on the step's dependent chain.
                __builtin_amdgcn_sched_barrier(0);
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
                __builtin_amdgcn_sched_barrier(0);
                const bf16x4 Ub = pack4(G::UW ? (Ua + Uc) + u0w : Ua + Uc);
                *reinterpret_cast<bf16x4 *>(ex + 4096 + lane * 8) = Ub;
#pragma unroll
                for (int m = 0; m < 8; ++m) S[m] = mma_k16(kd[m], Ub, S[m]);
            };
            bf16x8 wnA[4], wnB[4];
            bf16x4 kdA[8], kdB[8];
            f32x4 u0A, u0B;
            float gvA[2], gvB[2];
            barrier_lds();  // B_-1
            load(stage(0), j0, wnA, kdA, u0A, gvA);
            int64_t j = 0;
            for (; j + 1 < J; j += 2) {
                step(j, wnA, kdA, u0A, gvA, wnB, kdB, u0B, gvB);
                step(j + 1, wnB, kdB, u0B, gvB, wnA, kdA, u0A, gvA);
            }
            if (j < J) step(j, wnA, kdA, u0A, gvA, wnB, kdB, u0B, gvB);
            barrier_lds();  // B_J
        }
        store_state_tile(S, pw.sout, pw.sout_row, pw.sout16, col, g4);
        return;
    }

    // ---------------- output: O = Q~ S + P U of step j - 1
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
            const int64_t ja = j0 + jo;  // sub-chunk of the sequence
            __bf16 *orow = ob + (size_t)(16 * ja) * tokstride;
            if (16 * ja + 16 <= L) {  // the whole sub-chunk lies in the sequence
#pragma unroll
                for (int i = 0; i < 4; ++i) (orow + (size_t)i * tokstride)[loff] = (__bf16)O[i];
            } else {
                const int64_t r0 = 16 * ja + 4 * g4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (r0 + i < L) (orow + (size_t)i * tokstride)[loff] = (__bf16)O[i];
            }
        }
    }
}

// Pass B for many (sequence, head) pairs: one workgroup per pair covering all 128
// dv columns, so each record crosses HBM and LDS once.  kRW recurrence waves hold
// two 16-column tiles of the state each (64 fp32 per lane) and also form the
// output of their columns; NP producer waves fill an NS-stage ring of whole
// records with the raw v rows of the head.  With enough pairs to fill every compute unit, per-step latency is
// hidden by the other workgroups' memory traffic and the kernel streams the
// records at the bandwidth the workgroups can draw, so the output products that
// a separate wave would take off the recurrence's chain stay in the same wave
// and no exchange area is needed.
struct WideGeom {
    static constexpr int kVRow = 2 * kHeadDim;                   // bytes of a raw v row
    static constexpr int kVInst = (19 * kVRow + 1023) / 1024;    // DMA instructions of the v rows
    static constexpr int kVOff = kRecArea;
    static constexpr int kStage = kRecArea + kVInst * 1024;
    static constexpr int kInst = kRecInst + kVInst;              // DMA instructions per stage
    static constexpr int NP = KDA_SCAN_PRODUCERS;
    static constexpr int inst_of(int pw) { return (kInst + NP - 1 - pw) / NP; }
    static constexpr int kInstP0 = (kInst + NP - 1) / NP;  // inst_of(0)
    static constexpr int kRW = 4;                          // recurrence waves, two tiles each
    static constexpr int kWaves = kRW + NP;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int NSfit = 163840 / kStage;
    static constexpr int NS = NSfit < 10 ? NSfit : 10;
    static constexpr int kLds = NS * kStage;
    static constexpr int kMaxLater = NS - 3;
    static_assert(kStage % 1024 == 0, "stages move in whole DMA KiB");
    static_assert(2 * kRW * 16 == kHeadDim, "the recurrence waves cover every dv column");
    static_assert(NS >= 4, "the ring holds the stages of steps j - 1, j, j + 1 and the refill");
    static_assert(kInstP0 * kMaxLater < 64, "in-flight DMA exceeds the vmcnt range");
    static_assert(NP >= 1 && NP <= 8 && kWaves <= 16, "producers");
};

// Barriers as in scan_kernel (B_-1, then B_j for j = 0 .. J; at B_j stage j + 1
// is in LDS, and after it the producers refill the slot of stage j - 2).  During
// step j the recurrence waves compute step j from registers read from stage j
// and read stage j + 1.
template <bool SILU>
__global__ void __launch_bounds__(WideGeom::kThreads, 1) scan_wide_kernel(SplitParams p) {
    typedef WideGeom G;
    constexpr int D = kHeadDim, NS = G::NS;
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int pr = blockIdx.x;
    if (pr >= p.pairs) return;  // whole workgroup: no barrier is left waiting
    const int H = p.H;
    const int rk = pr / H, h = pr - rk * H;
    int n = rk;
    if (order_by_length(p)) {
        // the ring's first bytes as scratch, before any wave writes the ring
        n = seq_of_rank<G::kThreads>(p.cu, p.num_seqs, rk, reinterpret_cast<int *>(ring));
        __syncthreads();
    }
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup: no barrier is left waiting
    PairWork pw;
    if (!pair_work(p, n, h, slot, pw)) return;  // whole workgroup: no barrier is left waiting
    const int64_t s0 = pw.s0, L = pw.L, j0 = pw.j0, J = pw.steps;
    const unsigned char *rec0 = pw.rec0;

    if (w >= G::kRW) {
        // ---------------- producers (bare barriers: a fence would drain the DMA)
        if (J == 0) return;
        const VRows vr{reinterpret_cast<const unsigned char *>(p.v) + ((size_t)s0 * H + h) * D * 2,
                       (int64_t)H * D * 2, (int)L};
        producer_dispatch<G>(w - G::kRW, ring, rec0, vr, j0, lane, (int)J);
        return;
    }

    // ---------------- recurrence and output on tiles 2w, 2w + 1 (columns 32w ..)
    //   U = U0 - W S,  O = Q~ S + P U,  S = diag(gam) S + Kd^T U
    // S[t][m] holds rows 16 m + 4 g4 + i of column col[t] (accumulator layout).
    int col[2];
    col[0] = 32 * w + m16;
    col[1] = 32 * w + 16 + m16;
    f32x4 S[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) load_state_tile(S[t], pw.sin, pw.sin_row, pw.sin16, col[t], g4);
    if (J > 0) {
        const int64_t tokstride = (int64_t)H * D;
        __bf16 *ob = reinterpret_cast<__bf16 *>(p.o) + ((size_t)s0 * tokstride + (size_t)h * D);
        const uint32_t loff = (uint32_t)col[0] + 4u * (uint32_t)g4 * (uint32_t)tokstride;
        int rslot = 1 % NS;  // ring slot of stage j + 1 during step j
        constexpr bool silu = SILU;
        VConv vc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) load_vconv(p, slot, h, col[t], j0 == 0, vc[t]);
        struct Ops {
            bf16x8 wn[4], qg[4];
            bf16x4 kd[8], pp;
            f32x4 u0[2];
            float gv[2];
        };
        auto load = [&](const unsigned char *st, int64_t jabs, Ops &o) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o.wn[t] = *reinterpret_cast<const bf16x8 *>(st + R_WN + (t * 64 + lane) * 16);
                o.qg[t] = *reinterpret_cast<const bf16x8 *>(st + R_QG + (t * 64 + lane) * 16);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m)
                o.kd[m] = *reinterpret_cast<const bf16x4 *>(st + R_KD + (m * 64 + lane) * 8);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                o.gv[q] = *reinterpret_cast<const float *>(
                    st + R_GAM + (64 * q + 16 * (m16 >> 2) + 4 * g4 + (m16 & 3)) * 4);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                o.u0[t] = u0_tile<G::kVOff, G::kVRow>(st, col[t] * 2, lane, jabs == 0, vc[t], silu);
            o.pp = *reinterpret_cast<const bf16x4 *>(st + R_PP + lane * 8);
        };
        auto step = [&](int64_t j, const Ops &c, Ops &nx) {
            barrier_lds();  // B_j
            __builtin_amdgcn_sched_barrier(0);
            // (past the last step this reads a stale stage: harmless)
            load(ring + rslot * G::kStage, j0 + j + 1, nx);
            rslot = rslot + 1 == NS ? 0 : rslot + 1;
            bf16x8 Sp[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) Sp[t][q] = join8(pack4(S[t][2 * q]), pack4(S[t][2 * q + 1]));
            f32x4 Ua[2], Uc[2], O[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                Ua[t] = c.u0[t];
                Uc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // four independent U chains (two per tile), then the output products
#pragma unroll
            for (int q = 0; q < 4; q += 2)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    Ua[t] = mma_k32(c.wn[q], Sp[t][q], Ua[t]);
                    Uc[t] = mma_k32(c.wn[q + 1], Sp[t][q + 1], Uc[t]);
                }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int t = 0; t < 2; ++t) O[t] = mma_k32(c.qg[q], Sp[t][q], O[t]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                decay_tile<0>(S[t][0], c.gv);
                decay_tile<1>(S[t][1], c.gv);
                decay_tile<2>(S[t][2], c.gv);
                decay_tile<3>(S[t][3], c.gv);
                decay_tile<4>(S[t][4], c.gv);
                decay_tile<5>(S[t][5], c.gv);
                decay_tile<6>(S[t][6], c.gv);
                decay_tile<7>(S[t][7], c.gv);
            }
            bf16x4 Ub[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) Ub[t] = pack4(Ua[t] + Uc[t]);
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int t = 0; t < 2; ++t) S[t][m] = mma_k16(c.kd[m], Ub[t], S[t][m]);
#pragma unroll
            for (int t = 0; t < 2; ++t) O[t] = mma_k16w(c.pp, Ub[t], O[t]);  // after K = 32 steps
            const int64_t ja = j0 + j;  // sub-chunk of the sequence
            __bf16 *orow = ob + (size_t)(16 * ja) * tokstride;
            if (16 * ja + 16 <= L) {  // the whole sub-chunk lies in the sequence
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        (orow + (size_t)i * tokstride)[loff + 16 * t] = (__bf16)O[t][i];
            } else {
                const int64_t r0 = 16 * ja + 4 * g4;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (r0 + i < L) (orow + (size_t)i * tokstride)[loff + 16 * t] = (__bf16)O[t][i];
            }
        };
        Ops A, B;
        barrier_lds();  // B_-1
        load(ring, j0, A);  // stage 0 sits in slot 0
        int64_t j = 0;
        for (; j + 1 < J; j += 2) {
            step(j, A, B);
            step(j + 1, B, A);
        }
        if (j < J) step(j, A, B);
        barrier_lds();  // B_J
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) store_state_tile(S[t], pw.sout, pw.sout_row, pw.sout16, col[t], g4);
}

// ---------------------------------------------------------------------------
// Fused schedule for many (sequence, head) pairs: one workgroup per pair over
// all 128 dv columns.  Four pass-A waves form the records of the pair's
// sub-chunks (sub-chunks a, a + 4, ... for wave a; the two-pass record) in an
// NS-slot ring in LDS, and four recurrence waves run pass B's steps on them
// (two 16-column tiles each, U0 from the raw v rows and the output included),
// so no record leaves the CU.
// Slot j mod NS holds sub-chunk j.  The waves hand slots over through LDS
// words instead of barriers (a pass-A task spans several steps):
//   ready[s]  = j + 1 once sub-chunk j's record is complete in slot s;
//   done[w]   = the number of records recurrence wave w has read into registers.
// Pass-A wave a waits for min_w done[w] >= j - NS + 1 before writing sub-chunk j;
// recurrence wave w waits for ready[j mod NS] >= j + 1 before reading it.  A
// wait that polls spin_limit times (kda_set_spin_limit; 2^22 by default) without
// success sets the abort word, after which no wave of the workgroup waits again:
// a broken hand-over yields wrong results and never a workgroup that does not end.
struct FusedGeom {
    static constexpr int NS = 5;                  // record slots
    static constexpr int kAW = 4, kRW = 4;        // pass-A waves, recurrence waves
    static constexpr int kThreads = 64 * (kAW + kRW);
    static constexpr int kSlot = (int)kRec;       // a record slot: the two-pass record
    static constexpr int kAOff = NS * kSlot;      // pass-A scratch, A_WAVE bytes per wave
    static constexpr int kConvOff = kAOff + kAW * A_WAVE;
    // gam (2^b_last per dk channel, 128 fp32) of sub-chunk j sits in entry j mod
    // kGamSlots of a ring of its own, read by the recurrence waves during step j.
    // Pass A rewrites that entry (for sub-chunk j + kGamSlots) once every done[w]
    // >= j + kGamSlots - NS + 1 = j + NS + 1, which a recurrence wave publishes at
    // the end of step j + NS - 1, after step j.
    static constexpr int kGamSlots = 2 * NS, kGamOff = kConvOff + kConvLdsBytes;
    static constexpr int kFlagOff = kGamOff + kGamSlots * 512;
    static constexpr int kReady = kFlagOff, kDone = kFlagOff + 32, kAbort = kFlagOff + 60;
    // workgroup order (sequence lengths, then the chosen sequence)
    static constexpr int kOrderOff = kFlagOff + 64;
    static constexpr int kLds = kOrderOff + 4 * (kOrderMax + 1);
    static_assert(NS >= kAW && NS <= 8, "every pass-A wave has a slot to fill; ready[] fits 32 bytes");
    static_assert(kSlot % 16 == 0 && kLds <= 163840, "LDS");
    static_assert(2 * kRW * 16 == kHeadDim, "the recurrence waves cover every dv column");
};

__device__ __forceinline__ int lds_word(const unsigned char *lds, int off) {
    return __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(reinterpret_cast<const int *>(lds + off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
__device__ __forceinline__ void lds_word_set(unsigned char *lds, int off, int v) {
    // every earlier LDS access of this wave completes first (lgkmcnt only: the
    // fence is restricted to LDS, so loads from memory stay in flight)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __hip_atomic_store(reinterpret_cast<int *>(lds + off), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void give_up(unsigned char *lds) {
    __hip_atomic_store(reinterpret_cast<int *>(lds + FusedGeom::kAbort), 1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_ready(unsigned char *lds, int64_t j, int limit) {
    const int off = FusedGeom::kReady + 4 * (int)(j % FusedGeom::NS);
    for (int it = 0;; ++it) {
        if (lds_word(lds, off) >= (int)j + 1 || lds_word(lds, FusedGeom::kAbort)) break;
        if (it >= limit) {
            give_up(lds);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void wait_slot_free(unsigned char *lds, int64_t j, int limit) {
    const int want = (int)j - FusedGeom::NS + 1;
    if (want <= 0) return;
    for (int it = 0;; ++it) {
        int m = lds_word(lds, FusedGeom::kDone);
#pragma unroll
        for (int w = 1; w < FusedGeom::kRW; ++w) {
            const int d = lds_word(lds, FusedGeom::kDone + 4 * w);
            m = d < m ? d : m;
        }
        if (m >= want || lds_word(lds, FusedGeom::kAbort)) break;
        if (it >= limit) {
            give_up(lds);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <bool SILU>
__global__ void __launch_bounds__(FusedGeom::kThreads, 1) fused_kernel(SplitParams p) {
    typedef FusedGeom G;
    constexpr int D = kHeadDim, NS = G::NS;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_f[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int pr = blockIdx.x;
    if (pr >= p.pairs) return;  // whole workgroup
    const int H = p.H;
    const int rk = pr / H, h = pr - rk * H;
    const int n = order_by_length(p)
                      ? seq_of_rank<G::kThreads>(p.cu, p.num_seqs, rk, reinterpret_cast<int *>(smem_f + G::kOrderOff))
                      : rk;
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup
    int64_t s0, L;
    seq_bounds(p.cu, p.total, p.num_seqs, n, s0, L);
    const int64_t J = (L + 15) / 16;
    if (threadIdx.x < 16) reinterpret_cast<int *>(smem_f + G::kFlagOff)[threadIdx.x] = 0;
    {
        // the head's q, k, v conv taps and biases into LDS for the pass-A waves
        float *cwl = reinterpret_cast<float *>(smem_f + G::kConvOff);
        for (int i = threadIdx.x; i < 3 * 128; i += G::kThreads) {
            const int t = i >> 7, c = i & 127, ch = t * H * D + h * D + c;
            *reinterpret_cast<f32x4 *>(cwl + 4 * i) = *reinterpret_cast<const f32x4 *>(p.w + 4 * ch);
            cwl[3 * 128 * 4 + i] = p.bias ? p.bias[ch] : 0.f;
        }
    }
    __syncthreads();

    if (w >= G::kRW) {
        // ---------------- pass A: sub-chunks a, a + 4, ... into slot j mod NS
        const int a = w - G::kRW;
        if (a >= J) return;
        unsigned char *scratch = smem_f + G::kAOff + a * A_WAVE;
        const float *cwl = reinterpret_cast<const float *>(smem_f + G::kConvOff);
        ConvW unused;  // the fused body reads its taps from LDS
        SubTask t0;
        t0.slot = 0; t0.s0 = s0; t0.L = L; t0.n = n;
        // Software-pipelined over the wave's sub-chunks j = a, a + 4, ..: the loads
        // of sub-chunk j are issued first, the tail of sub-chunk j - 4 (from the
        // wave's tiles) runs while they are in flight, then the head of j consumes
        // them.  No row register lives across an iteration, so none is copied at
        // the loop's end while its load is still in flight.
        EarlyRows er;
        LateRows lr;
        float brl[4];
        t0.j = a;
        auto head = [&](int64_t j) {
            intra_head<true>(p, scratch, smem_f + (int)(j % NS) * G::kSlot, t0, h, lane, er, lr, unused, cwl,
                             nullptr, er, lr, [&] { wait_slot_free(smem_f, j, p.spin_limit); },
                             reinterpret_cast<float *>(smem_f + G::kGamOff + (int)(j % G::kGamSlots) * 512), brl);
        };
        auto tail = [&](int64_t j) {
            intra_tail(scratch, smem_f + (int)(j % NS) * G::kSlot, lane, brl);
            lds_word_set(smem_f, G::kReady + 4 * (int)(j % NS), (int)j + 1);
        };
        load_early(p, t0, h, lane, er);
        load_late(p, t0, h, lane, lr);
        head(a);
        for (int64_t j = a + G::kAW; j < J; j += G::kAW) {
            t0.j = j;  // j >= 4: not the sequence's first sub-chunk
            load_early<false>(p, t0, h, lane, er);
            load_late<false>(p, t0, h, lane, lr);
            tail(j - G::kAW);
            // the head waits for the loads: keep the whole tail in front of it
            __builtin_amdgcn_sched_barrier(0);
            head(j);
        }
        tail(J - 1 - (J - 1 - a) % G::kAW);
        return;
    }

    // ---------------- recurrence and output on tiles 2w, 2w + 1 (columns 32w ..)
    //   U = U0 - W S,  O = Q~ S + P U,  S = diag(gam) S + Kd^T U
    int col[2];
    col[0] = 32 * w + m16;
    col[1] = 32 * w + 16 + m16;
    const size_t srow = (size_t)slot * H + h;
    const bool st16 = p.state_bf16 != 0;
    f32x4 S[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) load_state_tile(S[t], p.state_in, srow, st16, col[t], g4);
    if (J > 0) {
        const int64_t tokstride = (int64_t)H * D;
        __bf16 *ob = reinterpret_cast<__bf16 *>(p.o) + ((size_t)s0 * tokstride + (size_t)h * D);
        const uint32_t loff = (uint32_t)col[0] + 4u * (uint32_t)g4 * (uint32_t)tokstride;
        // U0 = X diag(beta) V per tile, from the width-4 conv of the raw v rows
        // 4 g4 - 3 .. 4 g4 + 3 of the sub-chunk in this lane's columns, loaded one
        // step ahead (vx[t][k]: raw bf16 of row 4 g4 - 3 + k, column col[t]).  In a
        // sequence's first and last sub-chunks the rows are clamped into the
        // sequence (X diag(beta) has zero columns for the rows past its end) and
        // the rows before its start come from the conv state (or are zeros).
        const float *cwl = reinterpret_cast<const float *>(smem_f + G::kConvOff);
        const int64_t rowbytes = (int64_t)H * D * 2;
        const unsigned char *vseq = reinterpret_cast<const unsigned char *>(p.v) + ((size_t)s0 * H + h) * D * 2;
        const int vlane = 4 * g4 * (int)rowbytes + 2 * col[0];
        constexpr bool silu = SILU;
        uint32_t vx[2][7];
        auto load_v = [&](int64_t jr) {
            if (jr == 0 || 16 * jr + 16 > L) {
                const int CCH = 3 * H * D;
                const __bf16 *cs = p.cs_in ? reinterpret_cast<const __bf16 *>(p.cs_in) + (size_t)slot * 3 * CCH : nullptr;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int k = 0; k < 7; ++k) {
                        const int64_t r = 16 * jr + 4 * g4 - 3 + k;
                        const int64_t rr = r < L ? r : L - 1;
                        if (r < 0)
                            vx[t][k] = cs ? *reinterpret_cast<const unsigned short *>(
                                                cs + (size_t)(r + 3) * CCH + 2 * H * D + h * D + col[t])
                                          : 0u;
                        else
                            vx[t][k] = *reinterpret_cast<const unsigned short *>(vseq + rr * rowbytes + 2 * col[t]);
                    }
            } else {
                // rows 16 jr - 3 .. 16 jr + 15, all inside the sequence
                const int64_t r0 = 16 * jr - 3;
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<unsigned char *>(vseq + r0 * rowbytes), 0, (int)(19 * rowbytes), 0x00020000);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int k = 0; k < 7; ++k)
                        vx[t][k] = __builtin_amdgcn_raw_buffer_load_b16(rs, vlane + 32 * t, k * (int)rowbytes, 0);
            }
        };
        auto u0_of = [&](int t, bf16x4 xb) {
            const int c = col[t];
            const f32x4 wv = *reinterpret_cast<const f32x4 *>(cwl + (2 * 128 + c) * 4);
            const float bv = cwl[3 * 128 * 4 + 2 * 128 + c];
            float x[7];
#pragma unroll
            for (int k = 0; k < 7; ++k) x[k] = __uint_as_float(vx[t][k] << 16);
            f32x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = fmaf(wv[0], x[i], bv);
                a = fmaf(wv[1], x[i + 1], a);
                a = fmaf(wv[2], x[i + 2], a);
                a = fmaf(wv[3], x[i + 3], a);
                y[i] = silu ? a * sigmoidf_dev(a) : a;
            }
            return mma_k16w(xb, pack4(y), f32x4{0.f, 0.f, 0.f, 0.f});
        };
        struct Ops {
            bf16x8 wn[4], qg[4];
            bf16x4 kd[8], pp, xb;
        };
        auto load = [&](int64_t jr, Ops &o) {
            wait_ready(smem_f, jr, p.spin_limit);
            const unsigned char *st = smem_f + (int)(jr % NS) * G::kSlot;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o.wn[t] = *reinterpret_cast<const bf16x8 *>(st + R_WN + (t * 64 + lane) * 16);
                o.qg[t] = *reinterpret_cast<const bf16x8 *>(st + R_QG + (t * 64 + lane) * 16);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m)
                o.kd[m] = *reinterpret_cast<const bf16x4 *>(st + R_KD + (m * 64 + lane) * 8);
            o.xb = *reinterpret_cast<const bf16x4 *>(st + R_XB + lane * 8);
            o.pp = *reinterpret_cast<const bf16x4 *>(st + R_PP + lane * 8);
        };
        auto step = [&](int64_t j, const Ops &c, Ops &nx) {
            if (j + 1 < J) load(j + 1, nx);
            bf16x8 Sp[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) Sp[t][q] = join8(pack4(S[t][2 * q]), pack4(S[t][2 * q + 1]));
            f32x4 Ua[2], Uc[2], O[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                Ua[t] = u0_of(t, c.xb);
                Uc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (j + 1 < J) load_v(j + 1);  // vx is free again
#pragma unroll
            for (int q = 0; q < 4; q += 2)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    Ua[t] = mma_k32(c.wn[q], Sp[t][q], Ua[t]);
                    Uc[t] = mma_k32(c.wn[q + 1], Sp[t][q + 1], Uc[t]);
                }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int t = 0; t < 2; ++t) O[t] = mma_k32(c.qg[q], Sp[t][q], O[t]);
            {
                // gam of this lane's rows 16 m + 4 g4 .. + 3 from its ring entry
                const unsigned char *gam = smem_f + G::kGamOff + (int)(j % G::kGamSlots) * 512 + 16 * g4;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const f32x4 gm = *reinterpret_cast<const f32x4 *>(gam + 64 * m);
#pragma unroll
                    for (int t = 0; t < 2; ++t) S[t][m] *= gm;
                }
            }
            bf16x4 Ub[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) Ub[t] = pack4(Ua[t] + Uc[t]);
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int t = 0; t < 2; ++t) S[t][m] = mma_k16(c.kd[m], Ub[t], S[t][m]);
#pragma unroll
            for (int t = 0; t < 2; ++t) O[t] = mma_k16w(c.pp, Ub[t], O[t]);  // after K = 32 steps
            __bf16 *orow = ob + (size_t)(16 * j) * tokstride;
            if (16 * j + 16 <= L) {  // the whole sub-chunk lies in the sequence
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        (orow + (size_t)i * tokstride)[loff + 16 * t] = (__bf16)O[t][i];
            } else {
                const int64_t r0 = 16 * j + 4 * g4;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (r0 + i < L) (orow + (size_t)i * tokstride)[loff + 16 * t] = (__bf16)O[t][i];
            }
            // records 0 .. j + 1 are in registers (or past the end): their slots are free
            lds_word_set(smem_f, G::kDone + 4 * w, (int)j + 2);
        };
        Ops A, B;
        load(0, A);
        load_v(0);
        int64_t j = 0;
        for (; j + 1 < J; j += 2) {
            step(j, A, B);
            step(j + 1, B, A);
        }
        if (j < J) step(j, A, B);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) store_state_tile(S[t], p.state_out, srow, st16, col[t], g4);
}

hipError_t launch_fused(const SplitParams &sp, hipStream_t s) {
    typedef FusedGeom G;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&fused_kernel<false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
        if (attr == hipSuccess)
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&fused_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    });
    if (attr != hipSuccess) return attr;
    const unsigned blocks = (unsigned)sp.pairs;
    if (sp.flags & KDA_F_SILU)
        hipLaunchKernelGGL(fused_kernel<true>, dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    else
        hipLaunchKernelGGL(fused_kernel<false>, dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    trace("fused_kernel grid=(%u) block=%d lds=%d slots=%d", blocks, G::kThreads, G::kLds, G::NS);
    return hipGetLastError();
}

hipError_t launch_scan_wide(const SplitParams &sp, hipStream_t s) {
    typedef WideGeom G;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_wide_kernel<false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
        if (attr == hipSuccess)
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_wide_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    });
    if (attr != hipSuccess) return attr;
    const unsigned blocks = (unsigned)sp.pairs;
    if (sp.flags & KDA_F_SILU)
        hipLaunchKernelGGL(scan_wide_kernel<true>, dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    else
        hipLaunchKernelGGL(scan_wide_kernel<false>, dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    trace("scan_wide_kernel grid=(%u) block=%d lds=%d ring=%d", blocks, G::kThreads, G::kLds, G::NS);
    return hipGetLastError();
}

template <int NTW>
hipError_t launch_scan(const SplitParams &sp, hipStream_t s) {
    typedef ScanGeom<NTW> G;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_kernel<NTW, false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
        if (attr == hipSuccess)
            attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_kernel<NTW, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    });
    if (attr != hipSuccess) return attr;
    const unsigned blocks = (unsigned)((sp.pairs + 7) / 8) * 8u * (unsigned)sp.tiles;
    if (sp.flags & KDA_F_SILU)
        hipLaunchKernelGGL((scan_kernel<NTW, true>), dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    else
        hipLaunchKernelGGL((scan_kernel<NTW, false>), dim3(blocks), dim3(G::kThreads), G::kLds, s, sp);
    trace("scan_kernel<%d> grid=(%u) block=%d lds=%d ring=%d", NTW, blocks, G::kThreads, G::kLds, G::NS);
    return hipGetLastError();
}

}  // namespace

size_t split_workspace_bytes(int64_t total_tokens, int num_seqs, int H) {
    return (size_t)H * (size_t)(total_tokens / 16 + num_seqs) * kRec;
}

size_t split_window_bytes(int num_seqs, int H, int64_t jw) {
    return (size_t)H * (size_t)num_seqs * (size_t)jw * kRec + split_carry_bytes(num_seqs, H);
}

size_t split_carry_bytes(int num_seqs, int H) {
    return (size_t)num_seqs * (size_t)H * kHeadDim * kHeadDim * sizeof(float);
}

namespace {
// The kernel parameters every schedule of this file shares.
SplitParams common_params(const kda_prefill_args *a) {
    SplitParams sp;
    sp.q = a->q; sp.k = a->k; sp.v = a->v; sp.gate = a->gate; sp.beta = a->beta;
    sp.w = a->conv_weight; sp.bias = a->conv_bias; sp.cs_in = a->conv_state_in;
    sp.state_in = a->state_in; sp.state_out = a->state_out; sp.o = a->o;
    sp.state_bf16 = (a->flags & KDA_F_STATE_BF16) ? 1 : 0;
    sp.slots = a->state_slots; sp.num_slots = a->num_slots;
    sp.cu = a->cu_seqlens; sp.ws = static_cast<unsigned char *>(a->workspace);
    sp.total = a->total_tokens;
    sp.num_seqs = a->num_seqs; sp.H = a->num_heads;
    sp.scale = a->scale; sp.lb = a->gate_lower_bound; sp.flags = a->flags;
    sp.pairs = a->num_seqs * a->num_heads;
    sp.a_heads_fast = 0;
    sp.a_stride = 0;
    sp.jw = 0;
    sp.win = 0;
    sp.carry = nullptr;
    sp.nslots = 0;
    sp.tiles = 1;
    sp.spin_limit = spin_limit();
    return sp;
}
}  // namespace

hipError_t launch_prefill_fused(const kda_prefill_args *a, hipStream_t s) {
    return launch_fused(common_params(a), s);
}

hipError_t launch_prefill_split(const kda_prefill_args *a, int dv_tile, const SplitPlan &plan, hipStream_t s) {
    SplitParams sp = common_params(a);
    sp.jw = plan.jw;
    if (plan.jw > 0) {
        // records of one window first, then the carry
        sp.nslots = (int64_t)a->num_seqs * plan.jw;
        sp.carry = reinterpret_cast<float *>(sp.ws + (size_t)a->num_heads * (size_t)sp.nslots * kRec);
    } else {
        sp.nslots = a->total_tokens / 16 + a->num_seqs;
    }
    // 128 columns per workgroup: the wide pass B; otherwise at most two dv tiles of
    // 16 columns per workgroup
    const bool wide = dv_tile == kHeadDim;
    if (!wide && dv_tile > 32) dv_tile = 32;
    sp.tiles = kHeadDim / dv_tile;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&intra_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 4 * A_WAVE);
    });
    if (attr != hipSuccess) return attr;
    // two slots per wave: wave (x, w) owns slots x * 4 + w + k * 4 * gx and takes
    // the valid ones, so 8 * gx must cover every valid slot index.  Without windows
    // those are below ceil(total / 16) + num_seqs - 1 (the slot past a sequence's
    // last sub-chunk is never valid), which for one 16-aligned sequence is the
    // sub-chunk count itself and leaves no partly filled last round; with windows
    // they are the num_seqs * jw slots of a window.
    const int64_t span = plan.jw > 0 ? sp.nslots : (a->total_tokens + 15) / 16 + a->num_seqs - 1;
    const int64_t gx = (span + 7) / 8;
    sp.a_heads_fast = gx <= 65535;
    sp.a_stride = 4 * gx;
    const dim3 grid = sp.a_heads_fast ? dim3((unsigned)a->num_heads, (unsigned)gx)
                                      : dim3((unsigned)gx, (unsigned)a->num_heads);
    const int64_t windows = plan.jw > 0 ? plan.windows : 1;
    for (int64_t w = 0; w < windows; ++w) {
        sp.win = w;
        if (a->total_tokens > 0) {
            hipLaunchKernelGGL(intra_kernel, grid, dim3(256), 4 * A_WAVE, s, sp);
            trace("intra_kernel grid=(%u,%u) block=256 lds=%d window=%lld/%lld", grid.x, grid.y, 4 * A_WAVE,
                  (long long)w, (long long)windows);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipError_t e = wide ? launch_scan_wide(sp, s) : (dv_tile == 16 ? launch_scan<1>(sp, s) : launch_scan<2>(sp, s));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
