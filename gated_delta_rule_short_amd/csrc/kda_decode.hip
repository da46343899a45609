// kda_decode.hip -- recurrent decode of the KDA state: one token per call, a
// run of speculative tokens per call, and the commit of an accepted prefix.
//
// Source: "GLM-5.3-Flash im Detail" (flozi.net), section "Sequenz-Mixing":
// decoding one token is a recurrent update of the per-head matrix state (fp32,
// dk x dv = 128 x 128); conv of width four on q, k, v; channel-wise forget gate
// with log-decay >= -5; scalar-beta delta-rule write; the query reads the
// updated state.  Speculative verification ("GLM-5.3-Flash Internals", section
// "Serve rig": MTP with k = 5 drafted tokens) evaluates k + 1 tokens at once and
// keeps an accepted prefix.
//
// One workgroup of NT threads per (sequence, head).  A step is bound by HBM:
// the 64 KiB state is read once and written once.  Thread t owns columns
// 4*(t%32)..+3 of rows (t/32) + (NT/32)*m: every load instruction of a wave
// covers two whole 512-byte rows (fully coalesced float4 accesses), and the
// state values stay in registers between the read and the write.  Single-token
// decode uses NT = 512 (eight float4 per lane): the bare read-and-write-back of
// 1 GiB of states streams at 5.7 TB/s on this chip that way, against 5.2 TB/s
// with sixteen float4 per lane over 256 threads.  The multi-token verify and the
// commit keep NT = 256, the faster layout for their longer per-state work.
// The state loads are issued before the conv / L2 / gate prologue, so the
// prologue runs under the memory latency.  Per column j with decayed rows
// S'_i = alpha_i S_i:
//     a_j = sum_i S'_ij k_i,  c_j = sum_i S'_ij q_i
//     u_j = beta (v_j - a_j), o_j = scale (c_j + u_j (k . q)), S_ij = S'_ij + k_i u_j
// The row sums reduce across the two row groups of a wave (lane xor 32) and
// across the waves through LDS.
//
// The multi-token kernel runs that step for each of T tokens on the state held
// in registers and never writes it back; it writes per-token update records
// (alpha, normalised k, u and the raw conv inputs) instead.  A commit replays
// the first `accepted` records on the stored state.  Every helper below fixes
// its floating-point operation order (no contraction left to the compiler), so
// the replay and the multi-token outputs equal those of single-token decode bit
// for bit.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int D = kHeadDim;
constexpr int kMaxSpec = KDA_MAX_SPEC_TOKENS;

// Thread layout of the state for NT threads per (sequence, head).
template <int NT> struct Lay {
    static constexpr int kWaves = NT / 64;
    static constexpr int kRowStep = NT / 32;  // rows between a thread's state rows
    static constexpr int kRows = D / kRowStep;  // state rows (float4 each) per thread
    static_assert(kRows * kRowStep == D && 2 * D <= NT, "thread layout of the state");
};
constexpr int kDecodeThreads = 512;  // single-token decode
constexpr int kMultiThreads = 256;   // multi-token verify and commit
constexpr int kRec = KDA_UPDATE_FLOATS;  // floats per (sequence, head, token) record
static_assert(KDA_UPDATE_FLOATS == 6 * kHeadDim, "record = six rows of dk");

__device__ __forceinline__ f32x4 fma4(f32x4 a, float b, f32x4 c) {
    return f32x4{fmaf(a.x, b, c.x), fmaf(a.y, b, c.y), fmaf(a.z, b, c.z), fmaf(a.w, b, c.w)};
}

// Causal conv of width four: taps 0..2 weigh the three previous raw tokens
// (oldest first), tap 3 the current one.
__device__ __forceinline__ float conv4(const float *wc, float bias, float h0, float h1, float h2,
                                       float x, bool silu) {
#pragma clang fp contract(off)
    float y = fmaf(wc[3], x, fmaf(wc[2], h2, fmaf(wc[1], h1, fmaf(wc[0], h0, bias))));
    if (silu) y = y * sigmoidf_dev(y);
    return y;
}

// Per-row decay exp(g) of the channel-wise gate, g >= lb.
__device__ __forceinline__ float gate_alpha(float a, float lb, bool glog) {
#pragma clang fp contract(off)
    const float g = glog ? fmaxf(a, lb) : lb * sigmoidf_dev(a);
    return __expf(g);
}

// L2 scales of q and k and the normalised k . q from the two half sums of
// |q|^2, |k|^2, q . k held in red[wave][0..2].
__device__ __forceinline__ void norm_scales(const float (*red)[3], bool l2, float &iq, float &ik,
                                            float &kq) {
#pragma clang fp contract(off)
    const float sqq = red[0][0] + red[1][0];
    const float skk = red[0][1] + red[1][1];
    const float sqk = red[0][2] + red[1][2];
    iq = l2 ? rsqrtf(sqq + 1e-6f) : 1.f;
    ik = l2 ? rsqrtf(skk + 1e-6f) : 1.f;
    kq = sqk * iq * ik;
}

// One token on this thread's slice of the state (rows (tid/32) + (NT/32) m,
// columns 4 (tid%32)..+3).  sa, sk, sq: the token's decay, conv-ed key and query
// for all 128 rows, in LDS; with PRESCALED they already carry their L2 scales
// (ik, iq unused), else the step applies them (the same products either way).
// SCALED: the slice holds S~ = diag(c)^-1 S for the running decay product c of
// the call's tokens (c including this token's decay): sk and sq then hold c k
// and c q, and sa holds k / c, so that S'^T k = S~^T (c k), S'^T q = S~^T (c q)
// and the write is S~ += (k / c) u^T; the decay costs no multiply per element.
// vv: this thread's four v.  part: LDS for the cross-wave partial sums.  With
// four waves every thread adds the partials itself (part must not be read by a
// previous step that some thread may still be in); with eight, wave 0 adds them
// once into `tot` behind a second barrier, and the two barriers make one buffer
// of each enough for consecutive calls.  Returns u; ov receives the output
// columns.
template <bool PRESCALED, int NT, bool SCALED = false>
__device__ __forceinline__ f32x4 token_step(f32x4 (&st)[Lay<NT>::kRows], const float *sa, const float *sk,
                                            const float *sq, f32x4 vv, float ik, float iq, float kq,
                                            float beta, float scale, f32x4 (*part)[32][2],
                                            f32x4 (*tot)[2], int tid, f32x4 &ov) {
#pragma clang fp contract(off)
    typedef Lay<NT> LY;
    const int cg = tid & 31, rg = tid >> 5, wave = tid >> 6;
    f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
    float krow[LY::kRows];
#pragma unroll
    for (int m = 0; m < LY::kRows; ++m) {
        const int r = rg + LY::kRowStep * m;
        const float kr = PRESCALED ? sk[r] : sk[r] * ik;
        const float qr = PRESCALED ? sq[r] : sq[r] * iq;
        if constexpr (SCALED) {
            krow[m] = sa[r];
        } else {
            krow[m] = kr;
            st[m] = st[m] * sa[r];
        }
        ak = fma4(st[m], kr, ak);
        aq = fma4(st[m], qr, aq);
    }
    // the two row groups of the wave (lanes l and l ^ 32): one lane swap per
    // column leaves S'^T k sums in the low half and S'^T q sums in the high half
    f32x4 red;
#pragma unroll
    for (int e = 0; e < 4; ++e) red[e] = swap32_sum(ak[e], aq[e]);
    part[wave][cg][(tid >> 5) & 1] = red;
    barrier_lds();
    f32x4 s_k, s_q;
    if constexpr (LY::kWaves <= 4) {
        s_k = part[0][cg][0];
        s_q = part[0][cg][1];
#pragma unroll
        for (int w = 1; w < LY::kWaves; ++w) {
            s_k = s_k + part[w][cg][0];
            s_q = s_q + part[w][cg][1];
        }
    } else {
        // wave 0 adds the waves' partials in wave order (lanes 0..31 the k sums,
        // 32..63 the q sums of column group cg) once for the whole workgroup
        if (wave == 0) {
            const int half = tid >> 5;
            f32x4 acc = part[0][cg][half];
#pragma unroll
            for (int w = 1; w < LY::kWaves; ++w) acc = acc + part[w][cg][half];
            tot[cg][half] = acc;
        }
        barrier_lds();
        s_k = tot[cg][0];
        s_q = tot[cg][1];
    }
    const f32x4 u = beta * (vv - s_k);
    ov = scale * (s_q + u * kq);
#pragma unroll
    for (int m = 0; m < LY::kRows; ++m) st[m] = fma4(u, krow[m], st[m]);
    return u;
}

// Replays one update record on this thread's slice: S <- diag(alpha) S + k u^T,
// in the operation order token_step uses.
template <int NT>
__device__ __forceinline__ void replay_token(f32x4 (&st)[Lay<NT>::kRows], const float *alpha, const float *kn,
                                             f32x4 u, int tid) {
#pragma clang fp contract(off)
    const int rg = tid >> 5;
#pragma unroll
    for (int m = 0; m < Lay<NT>::kRows; ++m) {
        const int r = rg + Lay<NT>::kRowStep * m;
        st[m] = fma4(u, kn[r], st[m] * alpha[r]);
    }
}

// The state of one (sequence, head) moves between HBM and this thread's 16 x 4
// slice with non-temporal accesses: it is streamed exactly once each way, and
// must not displace the small, reused operands in L2.  SB is the storage type:
// fp32, or bf16 (widened exactly on load, rounded to nearest even on store).
template <int NT, typename SB>
__device__ __forceinline__ void load_state(f32x4 (&st)[Lay<NT>::kRows], const SB *S, int tid) {
    const int cg = tid & 31, rg = tid >> 5;
#pragma unroll
    for (int m = 0; m < Lay<NT>::kRows; ++m) {
        const SB *src = S + (size_t)(rg + Lay<NT>::kRowStep * m) * D + 4 * cg;
        if constexpr (sizeof(SB) == 4) {
            st[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
        } else {
            const uint64_t w = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(src));
            const uint32_t lo = (uint32_t)w, hi = (uint32_t)(w >> 32);
            st[m] = f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                          __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
        }
    }
}

template <int NT, typename SB>
__device__ __forceinline__ void store_state(const f32x4 (&st)[Lay<NT>::kRows], SB *S, int tid) {
    const int cg = tid & 31, rg = tid >> 5;
#pragma unroll
    for (int m = 0; m < Lay<NT>::kRows; ++m) {
        SB *dst = S + (size_t)(rg + Lay<NT>::kRowStep * m) * D + 4 * cg;
        if constexpr (sizeof(SB) == 4)
            __builtin_nontemporal_store(st[m], reinterpret_cast<f32x4 *>(dst));
        else
            __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, pack4(st[m])),
                                        reinterpret_cast<uint64_t *>(dst));
    }
}

__device__ __forceinline__ int clamp_count(int a, int hi) { return a < 0 ? 0 : (a > hi ? hi : a); }

// Conv window of one channel after a commit of `count` tokens: the last three
// raw tokens of (cache ++ the records' row `row`, tokens 0..count-1).  c0..c2:
// the cache as stored (oldest first); rec: the sequence-head's first record.
// The three record loads are issued together, before any is used.
__device__ __forceinline__ void committed_window(float c0, float c1, float c2, const float *rec,
                                                 int row, int ch, int count, float &h0, float &h1,
                                                 float &h2) {
    float r[3] = {0.f, 0.f, 0.f};  // raw tokens count-3 .. count-1 where they exist
#pragma unroll
    for (int j = 0; j < 3; ++j)
        if (count - 3 + j >= 0) r[j] = rec[(size_t)(count - 3 + j) * kRec + row * D + ch];
    h0 = count >= 3 ? r[0] : (count == 2 ? c2 : (count == 1 ? c1 : c0));
    h1 = count >= 2 ? r[1] : (count == 1 ? c2 : c1);
    h2 = count >= 1 ? r[2] : c2;
}

}  // namespace

struct DecodeParams {
    const void *q, *k, *v, *gate, *beta;
    const float *w, *bias;
    void *cs;
    void *state;  // fp32 or bf16 (SB)
    void *o;
    const int32_t *slots;  // pool row of each sequence (state, conv cache), or null
    int num_slots;
    int H;
    float scale, lb;
    uint32_t flags;
};

template <typename T, typename SB>
__global__ void __launch_bounds__(kDecodeThreads) decode_kernel(DecodeParams p) {
#pragma clang fp contract(off)
    constexpr int NTH = kDecodeThreads;
    typedef Lay<NTH> LY;
    const int pr = blockIdx.x;
    const int H = p.H;
    const int n = pr / H, h = pr - n * H;
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup, before any barrier
    const int tid = threadIdx.x;
    const int cg = tid & 31, rg = tid >> 5, wave = tid >> 6;

    __shared__ __attribute__((aligned(16))) float s_q[D], s_k[D], s_v[D], s_alpha[D];
    __shared__ float s_red[2][3];
    __shared__ f32x4 s_part[LY::kWaves][32][2];
    __shared__ f32x4 s_tot[32][2];

    // 1. issue the state loads (independent of the prologue).  The state is
    // streamed exactly once each way: non-temporal loads and stores keep it from
    // displacing the small, reused operands in L2.
    SB *S = reinterpret_cast<SB *>(p.state) + ((size_t)slot * H + h) * D * D;
    f32x4 st[LY::kRows];
    load_state<NTH>(st, S, tid);

    // 2. prologue: conv (and cache shift), L2 of q and k, gate
    const int CC = 3 * H * D;
    T *cs = reinterpret_cast<T *>(p.cs) + (size_t)slot * 3 * CC;
    const bool silu = p.flags & KDA_F_SILU;
    const bool l2 = !(p.flags & KDA_F_NO_QK_L2NORM);
    const bool glog = p.flags & KDA_F_GATE_IS_LOG;
    const size_t tok = (size_t)pr * D;  // offset of this (sequence, head) row
    auto conv = [&](const T *x, int ch) -> float {
        const float raw = to_f32(x[tok + (ch % D)]);
        const float h0 = to_f32(cs[ch]), h1 = to_f32(cs[CC + ch]), h2 = to_f32(cs[2 * CC + ch]);
        const float y = conv4(p.w + 4 * ch, p.bias ? p.bias[ch] : 0.f, h0, h1, h2, raw, silu);
        // shift the cache by one token (this workgroup alone owns these channels)
        cs[ch] = cs[CC + ch];
        cs[CC + ch] = cs[2 * CC + ch];
        cs[2 * CC + ch] = from_f32<T>(raw);
        return y;
    };
    // threads 0..127: q and k channel c; 128..255: v channel c and the gate of row
    // c; the others only hold state
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
    } else if (tid < 2 * D) {
        const int c = tid - D;
        s_v[c] = conv(reinterpret_cast<const T *>(p.v), 2 * H * D + h * D + c);
        s_alpha[c] = gate_alpha(to_f32(reinterpret_cast<const T *>(p.gate)[tok + c]), p.lb, glog);
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
    barrier_lds();
    float iq, ik, kq;
    norm_scales(s_red, l2, iq, ik, kq);
    const float beta = to_f32(reinterpret_cast<const T *>(p.beta)[pr]);

    // 3. decay, S'^T k and S'^T q, delta-rule value, output, write-back
    const f32x4 vv = *reinterpret_cast<const f32x4 *>(&s_v[4 * cg]);
    f32x4 ov;
    token_step<false, NTH>(st, s_alpha, s_k, s_q, vv, ik, iq, kq, beta, p.scale, s_part, s_tot, tid, ov);
    if (rg == 0) {
        T *o = reinterpret_cast<T *>(p.o) + tok + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(ov[e]);
    }
    store_state<NTH>(st, S, tid);
}

struct MultiParams {
    const void *q, *k, *v, *gate, *beta;
    const float *w, *bias;
    void *cs;
    void *state;          // fp32 or bf16 (SB)
    void *o;
    float *rec;           // [N][H][T][kRec] written
    const float *prec;    // pending records [N][H][pT][kRec] or null
    const int32_t *pacc;  // [N] pending accepted counts
    const int32_t *slots;  // pool row of each sequence (state, conv cache), or null
    int num_slots;
    int H, T, pT;
    float scale, lb;
    uint32_t flags;
};

// SCALED (see token_step): the tokens run on S~ = diag(c)^-1 S.  The host picks it
// only for the sigmoid gate with T (-lb) log2(e) <= 100, so that c >= 2^-100 and
// neither c nor 1 / c leaves the normal fp32 range.
template <typename T, typename SB, bool SCALED>
__global__ void __launch_bounds__(kMultiThreads) multi_kernel(MultiParams p) {
#pragma clang fp contract(off)
    constexpr int NTH = kMultiThreads, kThreads = NTH;
    typedef Lay<NTH> LY;
    const int pr = blockIdx.x;
    const int H = p.H, NT = p.T;
    const int n = pr / H, h = pr - n * H;
    const int slot = pool_slot(p.slots, p.num_slots, n);
    if (slot < 0) return;  // whole workgroup, before any barrier
    const int tid = threadIdx.x;
    const int cg = tid & 31, rg = tid >> 5, wave = tid >> 6;

    __shared__ __attribute__((aligned(16))) float s_q[kMaxSpec][D], s_k[kMaxSpec][D],
        s_v[kMaxSpec][D], s_alpha[kMaxSpec][D];
    __shared__ __attribute__((aligned(16))) float s_pend[kMaxSpec][3][D];
    __shared__ float s_red[kMaxSpec][2][3];
    __shared__ float s_beta[kMaxSpec];
    __shared__ f32x4 s_part[2][LY::kWaves][32][2];  // alternate tokens: one barrier per token

    // Every global load of the prologue is issued before any of them is used, so
    // the workgroup waits for memory once.  Threads 0..127 own q and k channel c,
    // threads 128..255 v channel c and the gate of row c; the others only hold
    // state (`act` is false for them: they take no part in the prologue).
    const bool act = tid < 2 * D;
    const bool qk = tid < D;
    const int c = qk ? tid : (act ? tid - D : 0);
    const int CC = 3 * H * D;
    const int ch0 = (qk ? 0 : 2 * H * D) + h * D + c;  // q or v channel
    const int ch1 = H * D + h * D + c;                  // k channel (q/k threads)
    const size_t tstride = (size_t)H * D;               // between tokens of a sequence
    const size_t base = ((size_t)n * NT * H + h) * D;   // token 0 of this (sequence, head)
    const T *src0 = reinterpret_cast<const T *>(qk ? p.q : p.v);
    const T *src1 = reinterpret_cast<const T *>(qk ? p.k : p.gate);
    T x0[kMaxSpec] = {}, x1[kMaxSpec] = {};
#pragma unroll
    for (int t = 0; t < kMaxSpec; ++t) {
        if (act && t < NT) {
            x0[t] = src0[base + t * tstride + c];
            x1[t] = src1[base + t * tstride + c];
        }
    }
    T *cs = reinterpret_cast<T *>(p.cs) + (size_t)slot * 3 * CC;
    T cr0[3] = {};
    if (act) {
        cr0[0] = cs[ch0];
        cr0[1] = cs[CC + ch0];
        cr0[2] = cs[2 * CC + ch0];
    }
    T cr1[3] = {};
    if (qk) {
        cr1[0] = cs[ch1];
        cr1[1] = cs[CC + ch1];
        cr1[2] = cs[2 * CC + ch1];
    }
    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(p.w + 4 * ch0);
    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(p.w + 4 * ch1);  // unused by v threads
    const float b0 = p.bias ? p.bias[ch0] : 0.f, b1 = p.bias ? p.bias[ch1] : 0.f;
    if (act && !qk && c < NT)
        s_beta[c] = to_f32(reinterpret_cast<const T *>(p.beta)[((size_t)n * NT + c) * H + h]);

    SB *S = reinterpret_cast<SB *>(p.state) + ((size_t)slot * H + h) * D * D;
    f32x4 st[LY::kRows];
    load_state<NTH>(st, S, tid);

    // pending commit: the accepted prefix of the previous call's records
    int na = 0;
    const float *prec = nullptr;
    if (p.prec) {
        na = clamp_count(p.pacc[n], p.pT);
        prec = p.prec + (size_t)pr * p.pT * kRec;
        constexpr int per = 3 * D / 4;  // float4 of rows 0..2 per record
        constexpr int kPend = (kMaxSpec * per + kThreads - 1) / kThreads;
        f32x4 pv[kPend];
#pragma unroll
        for (int j = 0; j < kPend; ++j) {
            const int i = tid + kThreads * j, t = i / per;
            if (i < na * per) pv[j] = reinterpret_cast<const f32x4 *>(prec + (size_t)t * kRec)[i - t * per];
        }
#pragma unroll
        for (int j = 0; j < kPend; ++j) {
            const int i = tid + kThreads * j, t = i / per;
            if (i < na * per) reinterpret_cast<f32x4 *>(&s_pend[t][0][0])[i - t * per] = pv[j];
        }
    }
    // conv windows after the pending commit (stored back when it moved them)
    float h0 = 0.f, h1 = 0.f, h2 = 0.f, g0 = 0.f, g1 = 0.f, g2 = 0.f;
    if (act)
        committed_window(to_f32(cr0[0]), to_f32(cr0[1]), to_f32(cr0[2]), prec, qk ? 3 : 5, c, na, h0,
                         h1, h2);
    if (qk)
        committed_window(to_f32(cr1[0]), to_f32(cr1[1]), to_f32(cr1[2]), prec, 4, c, na, g0, g1, g2);
    if (act && na > 0) {
        cs[ch0] = from_f32<T>(h0);
        cs[CC + ch0] = from_f32<T>(h1);
        cs[2 * CC + ch0] = from_f32<T>(h2);
        if (qk) {
            cs[ch1] = from_f32<T>(g0);
            cs[CC + ch1] = from_f32<T>(g1);
            cs[2 * CC + ch1] = from_f32<T>(g2);
        }
    }

    // conv of the T new tokens (and gates), raw inputs into rows 3..5 and decays
    // into row 0 of their records
    const bool silu = p.flags & KDA_F_SILU;
    const bool l2 = !(p.flags & KDA_F_NO_QK_L2NORM);
    const bool glog = p.flags & KDA_F_GATE_IS_LOG;
    const float wc0[4] = {w0.x, w0.y, w0.z, w0.w}, wc1[4] = {w1.x, w1.y, w1.z, w1.w};
    float *rec = p.rec + (size_t)pr * NT * kRec;
#pragma unroll
    for (int t = 0; t < kMaxSpec; ++t) {
        if (act && t < NT) {
            float *rt = rec + (size_t)t * kRec;
            const float r0 = to_f32(x0[t]);
            const float y0 = conv4(wc0, b0, h0, h1, h2, r0, silu);
            h0 = h1;
            h1 = h2;
            h2 = r0;
            if (qk) {
                const float r1 = to_f32(x1[t]);
                const float y1 = conv4(wc1, b1, g0, g1, g2, r1, silu);
                g0 = g1;
                g1 = g2;
                g2 = r1;
                s_q[t][c] = y0;
                s_k[t][c] = y1;
                rt[3 * D + c] = r0;
                rt[4 * D + c] = r1;
                const float a = wave_sum(y0 * y0), b = wave_sum(y1 * y1), e = wave_sum(y0 * y1);
                if ((tid & 63) == 0) {
                    s_red[t][wave][0] = a;
                    s_red[t][wave][1] = b;
                    s_red[t][wave][2] = e;
                }
            } else {
                const float al = gate_alpha(to_f32(x1[t]), p.lb, glog);
                s_v[t][c] = y0;
                s_alpha[t][c] = al;
                rt[5 * D + c] = r0;
                rt[c] = al;
            }
        }
    }
    barrier_lds();

    // apply the pending commit and store the committed state
    if (na > 0) {
        for (int t = 0; t < na; ++t)
            replay_token<NTH>(st, s_pend[t][0], s_pend[t][1],
                              *reinterpret_cast<const f32x4 *>(&s_pend[t][2][4 * cg]), tid);
        store_state<NTH>(st, S, tid);
    }
    // L2-normalised q and k of the new tokens, in place; k also into row 1 of
    // the records.  SCALED: c k, c q and k / c in place of k, q and the decay,
    // c the running product of the decays of row c over the tokens
    if (qk) {
        float cr = 1.f;
        for (int t = 0; t < NT; ++t) {
            float iq, ik, kq;
            norm_scales(s_red[t], l2, iq, ik, kq);
            const float kn = s_k[t][c] * ik;
            const float qn = s_q[t][c] * iq;
            rec[(size_t)t * kRec + D + c] = kn;
            if constexpr (SCALED) {
                cr = cr * s_alpha[t][c];
                s_k[t][c] = cr * kn;
                s_q[t][c] = cr * qn;
                s_alpha[t][c] = kn * __builtin_amdgcn_rcpf(cr);
            } else {
                s_k[t][c] = kn;
                s_q[t][c] = qn;
            }
        }
    }
    barrier_lds();

    // the T tokens in order, on the state held in registers
    T *ob = reinterpret_cast<T *>(p.o) + base + 4 * cg;
    for (int t = 0; t < NT; ++t) {
        float iq, ik, kq;
        norm_scales(s_red[t], l2, iq, ik, kq);
        const f32x4 vv = *reinterpret_cast<const f32x4 *>(&s_v[t][4 * cg]);
        f32x4 ov;
        const f32x4 u = token_step<true, NTH, SCALED>(st, s_alpha[t], s_k[t], s_q[t], vv, ik, iq, kq, s_beta[t],
                                              p.scale, s_part[t & 1], nullptr, tid, ov);
        if (rg == 0) {
            T *o = ob + t * tstride;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(ov[e]);
            *reinterpret_cast<f32x4 *>(rec + (size_t)t * kRec + 2 * D + 4 * cg) = u;
        }
    }
}

struct CommitParams {
    const int32_t *acc;
    const float *rec;
    void *cs;
    void *state;  // fp32 or bf16 (SB)
    const int32_t *slots;  // pool row of each sequence (state, conv cache), or null
    int num_slots;
    int H, T;
};

template <typename T, typename SB>
__global__ void __launch_bounds__(kMultiThreads) commit_kernel(CommitParams p) {
#pragma clang fp contract(off)
    constexpr int NTH = kMultiThreads, kThreads = NTH;
    typedef Lay<NTH> LY;
    const int pr = blockIdx.x;
    const int H = p.H;
    const int n = pr / H, h = pr - n * H;
    const int tid = threadIdx.x, cg = tid & 31;
    const int slot = pool_slot(p.slots, p.num_slots, n);
    const int na = clamp_count(p.acc[n], p.T);
    if (na == 0 || slot < 0) return;  // uniform over the workgroup

    __shared__ __attribute__((aligned(16))) float s_pend[kMaxSpec][3][D];
    SB *S = reinterpret_cast<SB *>(p.state) + ((size_t)slot * H + h) * D * D;
    f32x4 st[LY::kRows];
    load_state<NTH>(st, S, tid);
    const float *rec = p.rec + (size_t)pr * p.T * kRec;
    // every load below is issued before any is used: the records' alpha, k and u
    // rows (at most kPend float4 per thread), then this thread's conv channel
    // (i = tid of the head's 3 x 128: its cached taps and the raw rows of the last
    // three accepted tokens)
    constexpr int per = 3 * D / 4;
    constexpr int kPend = (kMaxSpec * per + kThreads - 1) / kThreads;
    constexpr int kConvPer = (3 * D + kThreads - 1) / kThreads;  // conv channels per thread
    f32x4 pv[kPend];
#pragma unroll
    for (int j = 0; j < kPend; ++j) {
        const int i = tid + kThreads * j, t = i / per;
        if (i < na * per) pv[j] = reinterpret_cast<const f32x4 *>(rec + (size_t)t * kRec)[i - t * per];
    }
    const int CC = 3 * H * D;
    T *cs = reinterpret_cast<T *>(p.cs) + (size_t)slot * 3 * CC;
    T cr[kConvPer][3];
    float hw[kConvPer][3];
#pragma unroll
    for (int q = 0; q < kConvPer; ++q) {
        const int i = tid + kThreads * q;
        if (i < 3 * D) {
            const int part = i / D, c = i - part * D;  // 0 q, 1 k, 2 v
            const int ch = part * H * D + h * D + c;
            cr[q][0] = cs[ch];
            cr[q][1] = cs[CC + ch];
            cr[q][2] = cs[2 * CC + ch];
            committed_window(to_f32(cr[q][0]), to_f32(cr[q][1]), to_f32(cr[q][2]), rec, 3 + part, c,
                             na, hw[q][0], hw[q][1], hw[q][2]);
        }
    }
#pragma unroll
    for (int j = 0; j < kPend; ++j) {
        const int i = tid + kThreads * j, t = i / per;
        if (i < na * per) reinterpret_cast<f32x4 *>(&s_pend[t][0][0])[i - t * per] = pv[j];
    }
#pragma unroll
    for (int q = 0; q < kConvPer; ++q) {
        const int i = tid + kThreads * q;
        if (i < 3 * D) {
            const int part = i / D, c = i - part * D;
            const int ch = part * H * D + h * D + c;
            cs[ch] = from_f32<T>(hw[q][0]);
            cs[CC + ch] = from_f32<T>(hw[q][1]);
            cs[2 * CC + ch] = from_f32<T>(hw[q][2]);
        }
    }
    barrier_lds();
    for (int t = 0; t < na; ++t)
        replay_token<NTH>(st, s_pend[t][0], s_pend[t][1],
                          *reinterpret_cast<const f32x4 *>(&s_pend[t][2][4 * cg]), tid);
    store_state<NTH>(st, S, tid);
}

// Launch of the instance for (token dtype, state storage): one workgroup of
// `threads` threads per (sequence, head).
template <typename P>
static void launch_typed(const char *name, int threads, kda_dtype dt, uint32_t flags, unsigned blocks,
                         const P &p, hipStream_t s, void (*bb)(P), void (*bf)(P), void (*fb)(P),
                         void (*ff)(P)) {
    const bool sb16 = flags & KDA_F_STATE_BF16;
    void (*k)(P) = dt == KDA_BF16 ? (sb16 ? bb : bf) : (sb16 ? fb : ff);
    hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, s, p);
    trace("%s<tokens %s, state %s> grid=(%u) block=%d lds=0", name, dt == KDA_BF16 ? "bf16" : "f32",
          sb16 ? "bf16" : "f32", blocks, threads);
}

hipError_t launch_decode(const kda_decode_args *a, hipStream_t s) {
    DecodeParams p;
    p.q = a->q; p.k = a->k; p.v = a->v; p.gate = a->gate; p.beta = a->beta;
    p.w = a->conv_weight; p.bias = a->conv_bias;
    p.cs = a->conv_state; p.state = a->state; p.o = a->o;
    p.slots = a->state_slots; p.num_slots = a->num_slots;
    p.H = a->num_heads;
    p.scale = a->scale; p.lb = a->gate_lower_bound; p.flags = a->flags;
    const unsigned blocks = (unsigned)a->num_seqs * (unsigned)a->num_heads;
    launch_typed<DecodeParams>("decode_kernel", kDecodeThreads, a->dtype, a->flags, blocks, p, s,
                     decode_kernel<__bf16, __bf16>, decode_kernel<__bf16, float>, decode_kernel<float, __bf16>, decode_kernel<float, float>);
    return hipGetLastError();
}

hipError_t launch_decode_multi(const kda_decode_multi_args *a, hipStream_t s) {
    MultiParams p;
    p.q = a->q; p.k = a->k; p.v = a->v; p.gate = a->gate; p.beta = a->beta;
    p.w = a->conv_weight; p.bias = a->conv_bias;
    p.cs = a->conv_state; p.state = a->state; p.o = a->o; p.rec = a->updates;
    p.prec = a->pending_updates; p.pacc = a->pending_accepted;
    p.slots = a->state_slots; p.num_slots = a->num_slots;
    p.H = a->num_heads; p.T = a->num_tokens; p.pT = a->pending_updates ? a->pending_tokens : 0;
    p.scale = a->scale; p.lb = a->gate_lower_bound; p.flags = a->flags;
    const unsigned blocks = (unsigned)a->num_seqs * (unsigned)a->num_heads;
    // the state in its scaled form when the decays of the T tokens keep their
    // product at or above 2^-100 (sigmoid gate: each decay is at least 2^(lb log2 e))
    const bool scaled = !(a->flags & KDA_F_GATE_IS_LOG) &&
                        (double)a->num_tokens * (double)(-a->gate_lower_bound) * 1.4426950408889634 <= 100.0;
    if (scaled)
        launch_typed<MultiParams>("multi_kernel<scaled>", kMultiThreads, a->dtype, a->flags, blocks, p, s,
                                  multi_kernel<__bf16, __bf16, true>, multi_kernel<__bf16, float, true>,
                                  multi_kernel<float, __bf16, true>, multi_kernel<float, float, true>);
    else
        launch_typed<MultiParams>("multi_kernel", kMultiThreads, a->dtype, a->flags, blocks, p, s,
                                  multi_kernel<__bf16, __bf16, false>, multi_kernel<__bf16, float, false>,
                                  multi_kernel<float, __bf16, false>, multi_kernel<float, float, false>);
    return hipGetLastError();
}

hipError_t launch_decode_commit(const kda_decode_commit_args *a, hipStream_t s) {
    CommitParams p;
    p.acc = a->accepted; p.rec = a->updates; p.cs = a->conv_state; p.state = a->state;
    p.slots = a->state_slots; p.num_slots = a->num_slots;
    p.H = a->num_heads; p.T = a->num_tokens;
    const unsigned blocks = (unsigned)a->num_seqs * (unsigned)a->num_heads;
    launch_typed<CommitParams>("commit_kernel", kMultiThreads, a->dtype, a->flags, blocks, p, s,
                     commit_kernel<__bf16, __bf16>, commit_kernel<__bf16, float>, commit_kernel<float, __bf16>, commit_kernel<float, float>);
    return hipGetLastError();
}

}  // namespace kda
