// kda_prefill.hip -- chunk-parallel KDA prefill on gfx950 matrix cores.
//
// Source: "GLM-5.3-Flash im Detail" (flozi.net), section "Sequenz-Mixing: 34
// KDA-Schichten mit festem Zustand": width-4 causal depthwise conv on q, k, v;
// a channel-wise forget gate (log-decay >= -5) attenuates a 128 x 128 fp32
// state per head; a scalar beta writes by the delta rule; the query reads the
// updated state; in prefill the tokens of a chunk are evaluated in parallel and
// a state is handed from chunk to chunk.
//
// Chunked form.  Inside a chunk of C = 16*NB tokens with state S0 on entry and
// b_r = sum_{t<=r} g_t (per channel, from the chunk start):
//     A_rs = sum_i k_ri k_si 2^(b_ri - b_si)   (s < r)     decayed key Gram
//     P_rs = sum_i q_ri k_si 2^(b_ri - b_si)   (s <= r)    decayed query-key Gram
//     X    = (I + diag(beta) A)^-1                          unit lower triangular
//     W    = X diag(beta) (K . 2^b),  U0 = X diag(beta) V
//     U    = U0 - W S0
//     O    = scale ((Q . 2^b) S0 + P U)
//     S1   = diag(2^b_last) S0 + (K . 2^(b_last - b))^T U
// which equals the token recurrence exactly in exact arithmetic.  Log-decays
// are kept in log2 units.
//
// Overflow-safe factoring.  A chunk's cumulative log-decay reaches -5*C (-320
// for C = 64), far below fp32's exponent range, so the Grams are formed on
// 16-row blocks with a reference point per block: with bl the cumsum inside
// a block (>= -80 since g >= -5 and 16 * 5 = 80 < ln(FLT_MAX) = 88.7) and G its
// total, the left factors k 2^bl, q 2^bl and the right factor k 2^(G - bl) are
// all <= 1; a diagonal block multiplies the right factor by 2^-G (<= 2^115 in
// log2 units, finite); an off-diagonal block (R, S) multiplies it by the decay
// 2^(B_R - B_{S+1}) of the blocks strictly between them (<= 1).
//
// Work split.  One workgroup of four waves per (sequence, head, dv tile); the
// fp32 state slice (128 x DVW) lives in registers in matrix-core accumulator
// layout for the whole sequence, so no state byte touches HBM between chunks.
// Per chunk:
//   1  wave R loads block R (+3 halo rows), convs, L2-normalises q and k, turns
//      the gate into log2-decays and their block cumsum        -> LDS
//   1b with the block totals of all waves, writes the MFMA operands -> LDS
//   2  decayed Grams A, P on 16 x 16 blocks (matrix cores); wave R inverts its
//      diagonal block of I + diag(beta) A by forward substitution (VALU, fp32)
//   3  block forward substitution for W (dk tiles spread over the waves) and
//      U0 (each wave its own dv tiles), chained in accumulator layout
//   4  per wave and dv tile: U, O, and the state update (matrix cores)
// Accumulator layout (16 x 16 tile): lane l holds column l % 16 and rows
// 4 (l / 16) + i.  Such a tile is consumed directly as the B operand of the
// next product with the K elements in the same slots, and the A operand is
// read from LDS with the matching K order, so the state, U, W and U0 chain
// between products in registers.
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mma.h"

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

struct PrefillParams {
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
    int64_t total;
    int num_seqs, H;
    float scale, lb;
    uint32_t flags;
    int pairs, tiles;
};

// Shared-memory layout (bytes).  E is the element type of the staged MFMA
// operands: bf16 for bf16 I/O, fp32 for fp32 I/O.  Row strides are padded so
// that the 16 rows read by one quarter-wave fall in distinct banks.
template <typename E, int NB, int DVW> struct Layout {
    static constexpr int C = 16 * NB;
    static constexpr int SRM = 128 + (sizeof(E) == 2 ? 4 : 2);  // [C][128]  token-major
    static constexpr int STR = C + 4;                            // [128][C]  channel-major
    static constexpr int SCC = C + 4;                            // [C][C]
    static constexpr int SXD = 20;                               // [16][16]
    static constexpr int NFO = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 1;
    static constexpr size_t RM = (size_t)C * SRM * sizeof(E);
    static constexpr size_t TR = (size_t)128 * STR * sizeof(E);
    static constexpr size_t KL = 0, QL = KL + RM, KR = QL + RM, QG = KR + RM;
    static constexpr size_t KGT = QG + RM, KDT = KGT + TR, VT = KDT + TR;
    static constexpr size_t LN = VT + (size_t)DVW * STR * sizeof(E);
    static constexpr size_t PM = LN + (size_t)C * SCC * sizeof(E);
    static constexpr size_t XD = PM + (size_t)C * SCC * sizeof(E);
    static constexpr size_t ND = XD + (((size_t)NB * 16 * SXD * sizeof(E) + 15) & ~(size_t)15);
    static constexpr size_t G2 = ND + (size_t)NB * 256 * 4;
    static constexpr size_t FD = G2 + (size_t)NB * 128 * 4;
    static constexpr size_t FO = FD + (size_t)NB * 128 * 4;
    static constexpr size_t GAM = FO + (size_t)NFO * 128 * 4;
    static constexpr size_t BET = GAM + 128 * 4;
    static constexpr int HS = 256 + DVW;  // halo row: q (128), k (128), v (DVW)
    static constexpr size_t HALO = BET + (((size_t)C * 4 + 15) & ~(size_t)15);
    static constexpr size_t TOTAL = HALO + (size_t)2 * 3 * HS * sizeof(E);
    // raw rows of the next chunk, staged by DMA into slots that are dead by then
    static constexpr size_t RQ = QL, RK = KR, RG = KGT, RV = VT, RB = ND;
    static_assert((size_t)C * SRM >= (size_t)C * 128 && (size_t)128 * STR >= (size_t)C * 128,
                  "staging fits");
};


// DMA of BYTES bytes (a multiple of 1 KiB) of row-gathered global data into
// contiguous LDS: 16-byte piece i comes from row (16 i) / ROW_BYTES of the
// source, byte (16 i) % ROW_BYTES.  Rows past `last_row` repeat it.  Each wave
// moves every fourth KiB; completion is tracked by vmcnt.
template <int ROW_BYTES, int BYTES>
__device__ __forceinline__ void dma_rows(unsigned char *lds_dst, const unsigned char *gbase,
                                         int64_t row_stride, int64_t first_row, int64_t last_row,
                                         int w, int lane) {
    static_assert(BYTES % 1024 == 0 && ROW_BYTES % 16 == 0, "DMA granularity");
#pragma unroll
    for (int inst = w; inst < BYTES / 1024; inst += 4) {
        const int piece = inst * 64 + lane;
        const int row = (piece * 16) / ROW_BYTES, col = (piece * 16) % ROW_BYTES;
        int64_t gr = first_row + row;
        gr = gr > last_row ? last_row : gr;
        __builtin_amdgcn_global_load_lds(gbase + gr * row_stride + col,
                                         (lds_void *)(lds_dst + inst * 1024), 16, 0, 0);
    }
}

// Index of the off-diagonal block pair (R, S), R >= S + 2, in the factor table.
__device__ __forceinline__ constexpr int fo_index(int R, int S) { return (R - 2) * (R - 1) / 2 + S; }

template <typename T, int NB, int DVW>
__global__ void __launch_bounds__(256, 1) prefill_kernel(PrefillParams p) {
    typedef T E;
    typedef Layout<E, NB, DVW> LY;
    typedef Ops<E> OP;
    typedef typename OP::B4 B4;
    constexpr int D = kHeadDim;
    constexpr int C = 16 * NB;
    constexpr int NTWG = DVW / 16;                // dv n-tiles per workgroup
    constexpr int WST = NTWG < 4 ? NTWG : 4;      // waves owning state columns
    constexpr int NTW = NTWG / WST;               // dv n-tiles per state wave
    constexpr int SRM = LY::SRM, STR = LY::STR, SCC = LY::SCC, SXD = LY::SXD, HS = LY::HS;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    E *sKL = reinterpret_cast<E *>(smem + LY::KL);  // also W (negated) after the Grams
    E *sQL = reinterpret_cast<E *>(smem + LY::QL);
    E *sKR = reinterpret_cast<E *>(smem + LY::KR);
    E *sQG = reinterpret_cast<E *>(smem + LY::QG);
    E *sKGT = reinterpret_cast<E *>(smem + LY::KGT);
    E *sKDT = reinterpret_cast<E *>(smem + LY::KDT);
    E *sVT = reinterpret_cast<E *>(smem + LY::VT);
    E *sLN = reinterpret_cast<E *>(smem + LY::LN);
    E *sPM = reinterpret_cast<E *>(smem + LY::PM);
    E *sXD = reinterpret_cast<E *>(smem + LY::XD);
    float *sNDT = reinterpret_cast<float *>(smem + LY::ND);  // diagonal blocks, transposed
    float *sG2 = reinterpret_cast<float *>(smem + LY::G2);
    float *sFD = reinterpret_cast<float *>(smem + LY::FD);
    float *sFO = reinterpret_cast<float *>(smem + LY::FO);
    float *sGAM = reinterpret_cast<float *>(smem + LY::GAM);
    float *sBET = reinterpret_cast<float *>(smem + LY::BET);
    E *sHALO = reinterpret_cast<E *>(smem + LY::HALO);
    const T *sRQ = reinterpret_cast<const T *>(smem + LY::RQ);
    const T *sRK = reinterpret_cast<const T *>(smem + LY::RK);
    const T *sRG = reinterpret_cast<const T *>(smem + LY::RG);
    const T *sRV = reinterpret_cast<const T *>(smem + LY::RV);
    float *sRB = reinterpret_cast<float *>(smem + LY::RB);
    E *sWN = sKL;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int m16 = lane & 15, g4 = lane >> 4;

    // All dv tiles of one (sequence, head) share blockIdx % 8, i.e. one XCD and
    // its L2, so the q/k/gate rows they all read are fetched from HBM once.
    const int bid = blockIdx.x;
    const int grp = bid / (8 * p.tiles), rem = bid - grp * 8 * p.tiles;
    const int tile = rem >> 3, pr = grp * 8 + (rem & 7);
    if (pr >= p.pairs) return;
    const int H = p.H;
    const int n = pr / H, h = pr - n * H;
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup, before any barrier
    const size_t spr = (size_t)slot * H + h;  // pool row of this (sequence, head)
    int64_t s0, L;
    seq_bounds(p.cu, p.total, p.num_seqs, n, s0, L);
    const int dvb = tile * DVW;
    const bool st_wave = w < WST;
    const int64_t tokstride = (int64_t)H * D;
    const bool silu = p.flags & KDA_F_SILU;
    const bool l2 = !(p.flags & KDA_F_NO_QK_L2NORM);
    const bool glog = p.flags & KDA_F_GATE_IS_LOG;
    const int CCH = 3 * H * D;

    // raw rows of chunk c -> LDS: q, k first (their slots die after the Grams),
    // gate, v and beta later (their slots die after the triangular solve)
    const unsigned char *gq = reinterpret_cast<const unsigned char *>(reinterpret_cast<const T *>(p.q) + (size_t)h * D);
    const unsigned char *gk = reinterpret_cast<const unsigned char *>(reinterpret_cast<const T *>(p.k) + (size_t)h * D);
    const unsigned char *gg = reinterpret_cast<const unsigned char *>(reinterpret_cast<const T *>(p.gate) + (size_t)h * D);
    const unsigned char *gv = reinterpret_cast<const unsigned char *>(reinterpret_cast<const T *>(p.v) + (size_t)h * D + dvb);
    const int64_t rstride = tokstride * (int64_t)sizeof(T);
    auto stage_qk = [&](int64_t c) {
        dma_rows<128 * sizeof(T), C * 128 * sizeof(T)>(smem + LY::RQ, gq, rstride, s0 + c * C, s0 + L - 1, w, lane);
        dma_rows<128 * sizeof(T), C * 128 * sizeof(T)>(smem + LY::RK, gk, rstride, s0 + c * C, s0 + L - 1, w, lane);
    };
    auto stage_rest = [&](int64_t c) {
        dma_rows<128 * sizeof(T), C * 128 * sizeof(T)>(smem + LY::RG, gg, rstride, s0 + c * C, s0 + L - 1, w, lane);
        dma_rows<DVW * sizeof(T), C * DVW * sizeof(T)>(smem + LY::RV, gv, rstride, s0 + c * C, s0 + L - 1, w, lane);
    };
    // beta of chunk c: one element per lane of wave 0, loaded early and parked in
    // LDS at the chunk boundary
    auto load_beta = [&](int64_t c) -> float {
        int64_t t = s0 + c * C + lane;
        t = t > s0 + L - 1 ? s0 + L - 1 : t;
        return to_f32(reinterpret_cast<const T *>(p.beta)[t * H + h]);
    };

    // fp32 state slice in accumulator layout: tile mt covers dk rows 16 mt..,
    // tile j the dv columns dvb + 16 (w NTW + j)..
    f32x4 S[8][NTW];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int col = dvb + 16 * (w * NTW + j) + m16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g4 + i;
                const size_t at = (spr * D + row) * D + col;
                S[mt][j][i] = !(st_wave && p.state_in) ? 0.f
                              : p.state_bf16 ? (float)reinterpret_cast<const __bf16 *>(p.state_in)[at]
                                             : reinterpret_cast<const float *>(p.state_in)[at];
            }
        }

    float beta_next = 0.f;
    if (L > 0) {
        stage_qk(0);
        stage_rest(0);
        if (w == 0 && lane < C) beta_next = load_beta(0);
    }
    // the strictly upper blocks of P are never written: zero them once
    for (int idx = tid; idx < C * SCC; idx += 256) sPM[idx] = from_f32<E>(0.f);
    // halo of the first chunk: the three raw rows before the sequence (conv state or zeros)
    {
        const T *csn = p.cs_in ? reinterpret_cast<const T *>(p.cs_in) + (size_t)slot * 3 * CCH : nullptr;
        E *hslot = sHALO + 1 * 3 * HS;  // read as the "previous" slot by chunk 0
        for (int idx = tid; idx < 3 * HS; idx += 256) {
            const int r = idx / HS, c = idx - r * HS;
            const int ch = c < 128 ? h * D + c : (c < 256 ? H * D + h * D + (c - 128)
                                                          : 2 * H * D + h * D + dvb + (c - 256));
            hslot[idx] = csn ? csn[(size_t)r * CCH + ch] : from_f32<E>(0.f);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (w == 0 && lane < C) sRB[lane] = beta_next;
    __syncthreads();

    const int64_t nchunks = (L + C - 1) / C;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t cbase = c * C;
        // ------------------------------------------------ phase 1: prologue
        float kl[16][2], ql[16][2], kr[16][2], vh[16][2], Gw[2] = {0.f, 0.f};
        const int c0 = 2 * lane;
        const bool has_v = c0 < DVW;
        if (w < NB) {
            const int R = w;
            const int64_t rowbase = cbase + 16 * R;
            const bool tail = rowbase + 16 > L;  // rows past the end in this block
            const E *hprev = sHALO + (int)((c + 1) & 1) * 3 * HS;
            const int vc = has_v ? c0 : 0;
            // raw rows 16R-3 .. 16R+15 of the chunk (the first three of block 0
            // come from the previous chunk or the conv state)
            float xq[19][2], xk[19][2], xv[19][2], ga[16][2];
#pragma unroll
            for (int r = 0; r < 19; ++r) {
                const int cr = 16 * R + r - 3;
                const T *rq = cr >= 0 ? sRQ + cr * 128 : hprev + (3 + cr) * HS;
                const T *rk = cr >= 0 ? sRK + cr * 128 : hprev + (3 + cr) * HS + 128;
                const T *rv = cr >= 0 ? sRV + cr * DVW : hprev + (3 + cr) * HS + 256;
                Pair<T>::load(rq + c0, xq[r][0], xq[r][1]);
                Pair<T>::load(rk + c0, xk[r][0], xk[r][1]);
                Pair<T>::load(rv + vc, xv[r][0], xv[r][1]);
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) Pair<T>::load(sRG + (16 * R + rr) * 128 + c0, ga[rr][0], ga[rr][1]);
            if (R == NB - 1) {  // keep the last three raw rows as the next chunk's halo
                E *hnext = sHALO + (int)(c & 1) * 3 * HS;
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    Pair<E>::store(hnext + r * HS + c0, xq[16 + r][0], xq[16 + r][1]);
                    Pair<E>::store(hnext + r * HS + 128 + c0, xk[16 + r][0], xk[16 + r][1]);
                    if (has_v) Pair<E>::store(hnext + r * HS + 256 + c0, xv[16 + r][0], xv[16 + r][1]);
                }
            }
            if (lane < 16) sBET[16 * R + lane] = rowbase + lane < L ? sRB[16 * R + lane] : 0.f;
            const int qch = h * D + c0, kch = H * D + h * D + c0, vch = 2 * H * D + h * D + dvb + vc;
            float wq[2][4], wk[2][4], wv[2][4], bq[2], bk[2], bv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                f32x4 a = *reinterpret_cast<const f32x4 *>(p.w + 4 * (qch + e));
                f32x4 b = *reinterpret_cast<const f32x4 *>(p.w + 4 * (kch + e));
                f32x4 cc = *reinterpret_cast<const f32x4 *>(p.w + 4 * (vch + e));
#pragma unroll
                for (int j = 0; j < 4; ++j) { wq[e][j] = a[j]; wk[e][j] = b[j]; wv[e][j] = cc[j]; }
                bq[e] = p.bias ? p.bias[qch + e] : 0.f;
                bk[e] = p.bias ? p.bias[kch + e] : 0.f;
                bv[e] = p.bias ? p.bias[vch + e] : 0.f;
            }
            // width-4 causal conv (tap 3 = current row)
            float yq[16][2], yk[16][2];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    yq[rr][e] = bq[e] + wq[e][0] * xq[rr][e] + wq[e][1] * xq[rr + 1][e] +
                                wq[e][2] * xq[rr + 2][e] + wq[e][3] * xq[rr + 3][e];
                    yk[rr][e] = bk[e] + wk[e][0] * xk[rr][e] + wk[e][1] * xk[rr + 1][e] +
                                wk[e][2] * xk[rr + 2][e] + wk[e][3] * xk[rr + 3][e];
                    vh[rr][e] = bv[e] + wv[e][0] * xv[rr][e] + wv[e][1] * xv[rr + 1][e] +
                                wv[e][2] * xv[rr + 2][e] + wv[e][3] * xv[rr + 3][e];
                }
            if (silu) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        yq[rr][e] *= sigmoidf_dev(yq[rr][e]);
                        yk[rr][e] *= sigmoidf_dev(yk[rr][e]);
                        vh[rr][e] *= sigmoidf_dev(vh[rr][e]);
                    }
            }
            // log2-decays of the gate
            float g2[16][2];
            if (glog) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                    for (int e = 0; e < 2; ++e) g2[rr][e] = fmaxf(ga[rr][e], p.lb) * kLog2e;
            } else {
                const float lb2 = p.lb * kLog2e;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
#pragma unroll
                    for (int e = 0; e < 2; ++e) g2[rr][e] = lb2 * sigmoidf_dev(ga[rr][e]);
            }
            if (tail) {  // rows past the end: no input, no decay
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
                    if (rowbase + rr >= L) {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            yq[rr][e] = 0.f; yk[rr][e] = 0.f; vh[rr][e] = 0.f; g2[rr][e] = 0.f;
                        }
                    }
            }
            // L2 norms of q and k: per-row sums over the 128 channels
            float rq[16], rk[16];
            if (l2) {
                float pq[16], pk[16], sq4[4], sk4[4];
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    pq[rr] = yq[rr][0] * yq[rr][0] + yq[rr][1] * yq[rr][1];
                    pk[rr] = yk[rr][0] * yk[rr][0] + yk[rr][1] * yk[rr][1];
                }
                rows16_sum(pq, sq4, lane);
                rows16_sum(pk, sk4, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sq4[j] = __builtin_amdgcn_rsqf(sq4[j] + 1e-6f);
                    sk4[j] = __builtin_amdgcn_rsqf(sk4[j] + 1e-6f);
                }
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    rq[rr] = row_value(sq4, rr);
                    rk[rr] = row_value(sk4, rr);
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) { rq[rr] = 1.f; rk[rr] = 1.f; }
            }
            // decays inside the block as running products of alpha = 2^g2:
            // eL_r = prod_{t<=r} alpha_t (<= 1), eR_r = prod_{t>r} alpha_t (<= 1)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float al[16], run = 1.f, gsum = 0.f;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    al[rr] = exp2_fast(g2[rr][e]);
                    gsum += g2[rr][e];
                    run *= al[rr];
                    const float qn = yq[rr][e] * rq[rr], kn = yk[rr][e] * rk[rr];
                    ql[rr][e] = qn * run;
                    kl[rr][e] = kn * run;
                    kr[rr][e] = kn;  // times eR below
                }
                float back = 1.f;
#pragma unroll
                for (int rr = 15; rr >= 0; --rr) {
                    kr[rr][e] *= back;
                    back *= al[rr];
                }
                Gw[e] = gsum;
                sG2[R * 128 + c0 + e] = gsum;
                sFD[R * 128 + c0 + e] = exp2_fast(-gsum);
            }
        }
        __syncthreads();

        // ------------------------------------ phase 1b: operands with block offsets
        if (w < NB) {
            const int R = w;
            float B2R[2] = {0.f, 0.f}, Bt[2] = {0.f, 0.f};
#pragma unroll
            for (int Rp = 0; Rp < NB; ++Rp)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float gsum = sG2[Rp * 128 + c0 + e];
                    if (Rp < R) B2R[e] += gsum;
                    Bt[e] += gsum;
                }
            float eB[2], eD[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                eB[e] = exp2_fast(B2R[e]);
                eD[e] = exp2_fast(Bt[e] - B2R[e] - Gw[e]);
            }
            float kgt[2][16], kdt[2][16], vtt[2][16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 16 * R + rr;
                const float bt = sBET[row];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    kgt[e][rr] = bt * kl[rr][e] * eB[e];
                    kdt[e][rr] = kr[rr][e] * eD[e];
                    vtt[e][rr] = bt * vh[rr][e];
                }
                Pair<E>::store(sKL + row * SRM + c0, kl[rr][0], kl[rr][1]);
                Pair<E>::store(sQL + row * SRM + c0, ql[rr][0], ql[rr][1]);
                Pair<E>::store(sKR + row * SRM + c0, kr[rr][0], kr[rr][1]);
                Pair<E>::store(sQG + row * SRM + c0, ql[rr][0] * eB[0], ql[rr][1] * eB[1]);
            }
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int o = (c0 + e) * STR + 16 * R + 4 * q4;
                    OP::store4(sKGT + o, kgt[e][4 * q4], kgt[e][4 * q4 + 1], kgt[e][4 * q4 + 2],
                               kgt[e][4 * q4 + 3]);
                    OP::store4(sKDT + o, kdt[e][4 * q4], kdt[e][4 * q4 + 1], kdt[e][4 * q4 + 2],
                               kdt[e][4 * q4 + 3]);
                    if (has_v)
                        OP::store4(sVT + o, vtt[e][4 * q4], vtt[e][4 * q4 + 1], vtt[e][4 * q4 + 2],
                                   vtt[e][4 * q4 + 3]);
                }
            if (R == 0) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    sGAM[c0 + e] = exp2_fast(Bt[e]);
#pragma unroll
                    for (int Ri = 2; Ri < NB; ++Ri)
#pragma unroll
                        for (int Si = 0; Si + 2 <= Ri; ++Si) {
                            float between = 0.f;
#pragma unroll
                            for (int Rp = Si + 1; Rp < Ri; ++Rp) between += sG2[Rp * 128 + c0 + e];
                            sFO[fo_index(Ri, Si) * 128 + c0 + e] = exp2_fast(between);
                        }
                }
            }
        }
        __syncthreads();

        // ----------------------------- phase 2: decayed Grams, diagonal inverses
        auto gram_tile = [&](int kind, int R, int Sb) {
            const E *lrow = (kind == 0 ? sKL : sQL) + (16 * R + m16) * SRM;
            const E *rrow = sKR + (16 * Sb + m16) * SRM;
            const float *f = (R == Sb) ? sFD + R * 128
                                       : (R >= Sb + 2 ? sFO + fo_index(R, Sb) * 128 : nullptr);
            const f32x4 acc = OP::gram(lrow, rrow, f, g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * g4 + i, sl = m16;
                float val = acc[i];
                if (kind == 0) {
                    if (R == Sb && sl >= rl) val = 0.f;
                    val *= sBET[16 * R + rl];
                    if (R == Sb) sNDT[R * 256 + sl * 16 + rl] = val;
                    else sLN[(16 * R + rl) * SCC + 16 * Sb + sl] = from_f32<E>(-val);
                } else {
                    if (R == Sb && sl > rl) val = 0.f;
                    sPM[(16 * R + rl) * SCC + 16 * Sb + sl] = from_f32<E>(val);
                }
            }
        };
        if (w < NB) {
            gram_tile(0, w, w);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < 16) {
                // column `lane` of (I + N)^-1, N the strictly lower diagonal block
                // (stored transposed): right-looking, so each step's updates are
                // independent of one another
                const float *Nt = sNDT + w * 256;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < 15; ++s) {
                    const float xs = x[s];
#pragma unroll
                    for (int i = s + 1; i < 16; ++i) x[i] -= Nt[s * 16 + i] * xs;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) sXD[(w * 16 + i) * SXD + lane] = from_f32<E>(x[i]);
            }
            gram_tile(1, w, w);
        }
        if constexpr (NB > 1) {
            constexpr int NOFF = NB * (NB - 1) / 2;
            for (int task = w; task < 2 * NOFF; task += 4) {
                const int kind = task / NOFF, idx = task - kind * NOFF;
                int R = 1, acc = 0;
                while (acc + R <= idx) { acc += R; ++R; }
                gram_tile(kind, R, idx - acc);
            }
        }
        __syncthreads();
        if (c + 1 < nchunks) stage_qk(c + 1);  // q, k slots are free from here on

        // ----------------------- phase 3: W and U0 by block forward substitution
        f32x4 U0[NB][NTW];
        {
            B4 Wb[2][NB];
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                const E *lnrow = sLN + (16 * R + m16) * SCC + 4 * g4;
                const E *xrow = sXD + (R * 16 + m16) * SXD + 4 * g4;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = 16 * (2 * w + j) + m16;
                    f32x4 rhs = OP::load4(sKGT + col * STR + 16 * R + 4 * g4);
                    rhs = OP::template chain<NB>(rhs, lnrow, Wb[j], R);
                    B4 rb[1] = {OP::pack(rhs)};
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 wr = OP::template chain<1>(z, xrow, rb, 1);
                    Wb[j][R] = OP::pack(wr);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sWN[(16 * R + 4 * g4 + i) * SRM + col] = from_f32<E>(-wr[i]);
                }
                if (st_wave) {
                    B4 Ub[NTW][NB];
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int col = 16 * (w * NTW + j) + m16;
                        f32x4 rhs = OP::load4(sVT + col * STR + 16 * R + 4 * g4);
#pragma unroll
                        for (int Rp = 0; Rp < R; ++Rp) Ub[j][Rp] = OP::pack(U0[Rp][j]);
                        rhs = OP::template chain<NB>(rhs, lnrow, Ub[j], R);
                        B4 rb[1] = {OP::pack(rhs)};
                        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                        U0[R][j] = OP::template chain<1>(z, xrow, rb, 1);
                    }
                }
            }
        }
        __syncthreads();
        if (c + 1 < nchunks) {  // gate, v, beta slots are free from here on
            stage_rest(c + 1);
            if (w == 0 && lane < C) beta_next = load_beta(c + 1);
        }

        // ----------------------------------------- phase 4: state path (per wave)
        if (st_wave) {
            B4 Sb[NTW][8];
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) Sb[j][mt] = OP::pack(S[mt][j]);
            B4 Ub[NTW][NB];
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                const E *wrow = sWN + (16 * R + m16) * SRM + 4 * g4;
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    Ub[j][R] = OP::pack(OP::template chain<8>(U0[R][j], wrow, Sb[j], 8));
            }
            const bool full = cbase + C <= L;
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                const E *qrow = sQG + (16 * R + m16) * SRM + 4 * g4;
                const E *prow = sPM + (16 * R + m16) * SCC + 4 * g4;
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    acc = OP::template chain<8>(acc, qrow, Sb[j], 8);
                    acc = OP::template chain<NB>(acc, prow, Ub[j], NB);
                    const int col = dvb + 16 * (w * NTW + j) + m16;
                    T *op = reinterpret_cast<T *>(p.o) + (size_t)(s0 + cbase + 16 * R + 4 * g4) * tokstride +
                            (size_t)h * D + col;
                    if (full) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) op[i * tokstride] = from_f32<T>(p.scale * acc[i]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (cbase + 16 * R + 4 * g4 + i < L)
                                op[i * tokstride] = from_f32<T>(p.scale * acc[i]);
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(sGAM + 16 * mt + 4 * g4);
                const E *krow = sKDT + (16 * mt + m16) * STR + 4 * g4;
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    S[mt][j] = OP::template chain<NB>(S[mt][j] * gam, krow, Ub[j], NB);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // next chunk's staged rows
        if (c + 1 < nchunks && w == 0 && lane < C) sRB[lane] = beta_next;
        __syncthreads();
    }

    if (st_wave && p.state_out) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int col = dvb + 16 * (w * NTW + j) + m16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t at = (spr * D + 16 * mt + 4 * g4 + i) * D + col;
                    if (p.state_bf16)
                        reinterpret_cast<__bf16 *>(p.state_out)[at] = (__bf16)S[mt][j][i];
                    else
                        reinterpret_cast<float *>(p.state_out)[at] = S[mt][j][i];
                }
            }
    }
}

template <typename T, int NB, int DVW>
static hipError_t launch_t(const PrefillParams &pp, hipStream_t s) {
    typedef Layout<T, NB, DVW> LY;
    static_assert(LY::TOTAL <= 160 * 1024, "shared memory budget");
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [] {
        attr_err = hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_kernel<T, NB, DVW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::TOTAL);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int groups = (pp.pairs + 7) / 8;
    const unsigned blocks = (unsigned)groups * 8u * (unsigned)pp.tiles;
    hipLaunchKernelGGL((prefill_kernel<T, NB, DVW>), dim3(blocks), dim3(256), LY::TOTAL, s, pp);
    trace("prefill_kernel<%s, chunk=%d, dv_tile=%d> grid=(%u) block=256 lds=%d",
          sizeof(T) == 2 ? "bf16" : "f32", 16 * NB, DVW, blocks, (int)LY::TOTAL);
    return hipGetLastError();
}

template <typename T, int NB>
static hipError_t dispatch_dv(const PrefillParams &pp, int dv_tile, hipStream_t s) {
    switch (dv_tile) {
        case 32: return launch_t<T, NB, 32>(pp, s);
        case 64: return launch_t<T, NB, 64>(pp, s);
        default: return launch_t<T, NB, 128>(pp, s);
    }
}

hipError_t launch_prefill(const PrefillLaunch &L, hipStream_t s) {
    const kda_prefill_args *a = L.a;
    PrefillParams pp;
    pp.q = a->q; pp.k = a->k; pp.v = a->v; pp.gate = a->gate; pp.beta = a->beta;
    pp.w = a->conv_weight; pp.bias = a->conv_bias;
    pp.cs_in = a->conv_state_in;
    pp.state_in = a->state_in; pp.state_out = a->state_out;
    pp.state_bf16 = (a->flags & KDA_F_STATE_BF16) ? 1 : 0;
    pp.slots = a->state_slots; pp.num_slots = a->num_slots;
    pp.o = a->o;
    pp.cu = a->cu_seqlens;
    pp.total = a->total_tokens;
    pp.num_seqs = a->num_seqs; pp.H = a->num_heads;
    pp.scale = a->scale; pp.lb = a->gate_lower_bound; pp.flags = a->flags;
    pp.pairs = a->num_seqs * a->num_heads;
    pp.tiles = kHeadDim / L.dv_tile;
    if (a->dtype == KDA_BF16) {
        switch (L.chunk) {
            case 16: return dispatch_dv<__bf16, 1>(pp, L.dv_tile, s);
            case 32: return dispatch_dv<__bf16, 2>(pp, L.dv_tile, s);
            default: return dispatch_dv<__bf16, 4>(pp, L.dv_tile, s);
        }
    }
    switch (L.chunk) {
        case 16: return dispatch_dv<float, 1>(pp, L.dv_tile, s);
        default: return dispatch_dv<float, 2>(pp, L.dv_tile, s);
    }
}

}  // namespace kda
