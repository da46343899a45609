/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * sequence mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or helper with the HIP library, and it
 * never touches a GPU.
 *
 * What it computes (source: "GLM-5.3-Flash im Detail" (flozi.net), section
 * "Sequenz-Mixing: 34 KDA-Schichten mit festem Zustand"; the same facts appear
 * on the "GLM-5.3-Flash Internals" dataset card, section "Anatomy"):
 *   - q, k and v each pass through a causal depthwise convolution of width 4;
 *   - a channel-wise forget gate, whose log-decay is bounded below at -5,
 *     attenuates the matrix state of every head;
 *   - a scalar beta drives a delta-rule write of v along k;
 *   - the query reads the *updated* state.
 * The recurrent state of one head is a dk x dv matrix held in fp32 by the
 * reference cache (same section, the 64x128x128 state arithmetic).
 *
 * Readings where the pages are silent (every one is an explicit argument or
 * flag so it can be changed in one place):
 *   - conv taps: cross-correlation, tap 3 multiplies the current token, the
 *     three taps before it the three previous tokens of the same sequence;
 *     positions before the sequence start come from conv_state_in (oldest
 *     first) or are zero; no activation unless ORACLE_SILU.
 *   - q and k (not v) are L2-normalised per head after the conv:
 *     x / sqrt(sum x^2 + 1e-6); ORACLE_NO_QK_L2NORM turns it off.
 *   - the gate input is the pre-activation a; log-decay g = lb * sigmoid(a)
 *     with lb = gate_lower_bound (-5), so g lies in (lb, 0);
 *     ORACLE_GATE_IS_LOG takes g = max(a, lb) instead.
 *   - the decay multiplies the dk rows of S[dk][dv]; order per token:
 *     decay, delta error against the decayed state, write, read.
 *   - scale is passed in (default 1/sqrt(dk) is chosen by the caller).
 *
 * Per token t of a sequence, per head (all fp64):
 *     S   <- diag(exp(g_t)) S
 *     u   =  beta_t * (v_t - S^T k_t)
 *     S   <- S + k_t u^T
 *     o_t =  scale * S^T q_t
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_SILU 1u
#define ORACLE_NO_QK_L2NORM 2u
#define ORACLE_GATE_IS_LOG 4u

#define L2_EPS 1e-6

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Value of conv channel `ch` at sequence position p (may be -3..-1). */
static double hist_value(const double *x, int64_t x_row_stride, int64_t x_col,
                         int64_t seq_start, int64_t p, const double *cs_in,
                         int64_t cs_channels, int64_t seq, int64_t ch)
{
    if (p >= 0)
        return x[(seq_start + p) * x_row_stride + x_col];
    if (cs_in == NULL)
        return 0.0;
    /* p = -3 is slot 0 (oldest), p = -1 is slot 2 (newest) */
    return cs_in[(seq * 3 + (3 + p)) * cs_channels + ch];
}

/* Width-4 causal depthwise conv of one channel at position p. */
static double conv_one(const double *x, int64_t x_row_stride, int64_t x_col,
                       int64_t seq_start, int64_t p, const double *w4,
                       const double *bias, const double *cs_in,
                       int64_t cs_channels, int64_t seq, int64_t ch, int silu)
{
    double y = bias ? bias[ch] : 0.0;
    for (int j = 0; j < 4; ++j)
        y += w4[j] * hist_value(x, x_row_stride, x_col, seq_start, p - 3 + j,
                                cs_in, cs_channels, seq, ch);
    if (silu)
        y = y * sigmoid(y);
    return y;
}

/* conv_state_out slot s after a sequence of length L: the last three raw
 * values of (conv_state_in ++ x[0..L)). */
static double tail_value(const double *x, int64_t x_row_stride, int64_t x_col,
                         int64_t seq_start, int64_t L, int s,
                         const double *cs_in, int64_t cs_channels, int64_t seq,
                         int64_t ch)
{
    int64_t p = L - 3 + s; /* sequence position of slot s */
    return hist_value(x, x_row_stride, x_col, seq_start, p, cs_in, cs_channels,
                      seq, ch);
}

/*
 * Standalone causal depthwise conv, width 4, over packed sequences.
 *   x, y          : [total_tokens][channels]
 *   weight        : [channels][4], tap 3 = current token
 *   bias          : [channels] or NULL
 *   conv_state_in : [num_seqs][3][channels] or NULL (zeros)
 *   conv_state_out: [num_seqs][3][channels] or NULL; may alias conv_state_in
 *   cu_seqlens    : [num_seqs + 1]
 */
void kda_oracle_short_conv(const double *x, double *y, int64_t total_tokens,
                           int64_t channels, const double *weight,
                           const double *bias, const double *conv_state_in,
                           double *conv_state_out, const int32_t *cu_seqlens,
                           int64_t num_seqs, int silu, int nthreads)
{
    (void)total_tokens;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
#else
    (void)nthreads;
#endif
    for (int64_t ch = 0; ch < channels; ++ch) {
        for (int64_t n = 0; n < num_seqs; ++n) {
            int64_t s0 = cu_seqlens[n], L = cu_seqlens[n + 1] - cu_seqlens[n];
            double tail[3];
            for (int s = 0; s < 3; ++s)
                tail[s] = tail_value(x, channels, ch, s0, L, s, conv_state_in,
                                     channels, n, ch);
            for (int64_t p = 0; p < L; ++p)
                y[(s0 + p) * channels + ch] =
                    conv_one(x, channels, ch, s0, p, weight + 4 * ch, bias,
                             conv_state_in, channels, n, ch, silu);
            if (conv_state_out)
                for (int s = 0; s < 3; ++s)
                    conv_state_out[(n * 3 + s) * channels + ch] = tail[s];
        }
    }
}

/*
 * Token-by-token KDA over packed sequences.
 *   q, k   : [total_tokens][H][dk]   raw (pre-conv)
 *   v      : [total_tokens][H][dv]   raw (pre-conv)
 *   gate   : [total_tokens][H][dk]   pre-activation a (or log-decay)
 *   beta   : [total_tokens][H]
 *   conv_w : [2*H*dk + H*dv][4]      channel order q, k, v; head-major inside
 *   conv_b : same channels, or NULL
 *   conv_state_in/out : [num_seqs][3][2*H*dk + H*dv] or NULL (out may alias in)
 *   state_in/out      : [num_seqs][H][dk][dv] or NULL (out may alias in)
 *   o      : [total_tokens][H][dv]
 */
void kda_oracle_prefill(int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                        const int32_t *cu_seqlens, const double *q,
                        const double *k, const double *v, const double *gate,
                        const double *beta, const double *conv_w,
                        const double *conv_b, const double *conv_state_in,
                        double *conv_state_out, const double *state_in,
                        double *state_out, double *o, double scale,
                        double gate_lower_bound, unsigned flags, int nthreads)
{
    const int64_t CC = 2 * H * dk + H * dv;
    const int silu = (flags & ORACLE_SILU) != 0;
    const int l2 = (flags & ORACLE_NO_QK_L2NORM) == 0;
    const int gate_is_log = (flags & ORACLE_GATE_IS_LOG) != 0;
    const int64_t pairs = num_seqs * H;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#else
    (void)nthreads;
#endif
    for (int64_t pr = 0; pr < pairs; ++pr) {
        const int64_t n = pr / H, h = pr % H;
        const int64_t s0 = cu_seqlens[n], L = cu_seqlens[n + 1] - cu_seqlens[n];
        double *S = (double *)calloc((size_t)(dk * dv), sizeof(double));
        double *qt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vt = (double *)malloc(sizeof(double) * (size_t)dv);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *ot = (double *)malloc(sizeof(double) * (size_t)dv);
        const int64_t qch = h * dk, kch = H * dk + h * dk, vch = 2 * H * dk + h * dv;

        if (state_in)
            memcpy(S, state_in + pr * dk * dv, sizeof(double) * (size_t)(dk * dv));

        for (int64_t p = 0; p < L; ++p) {
            const int64_t t = s0 + p;
            /* causal short conv on the raw q, k, v of this head */
            for (int64_t c = 0; c < dk; ++c) {
                qt[c] = conv_one(q, H * dk, h * dk + c, s0, p, conv_w + 4 * (qch + c),
                                 conv_b, conv_state_in, CC, n, qch + c, silu);
                kt[c] = conv_one(k, H * dk, h * dk + c, s0, p, conv_w + 4 * (kch + c),
                                 conv_b, conv_state_in, CC, n, kch + c, silu);
            }
            for (int64_t c = 0; c < dv; ++c)
                vt[c] = conv_one(v, H * dv, h * dv + c, s0, p, conv_w + 4 * (vch + c),
                                 conv_b, conv_state_in, CC, n, vch + c, silu);
            /* L2 normalisation of q and k over the head's dk channels */
            if (l2) {
                double sq = 0.0, sk = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    sq += qt[c] * qt[c];
                    sk += kt[c] * kt[c];
                }
                const double iq = 1.0 / sqrt(sq + L2_EPS), ik = 1.0 / sqrt(sk + L2_EPS);
                for (int64_t c = 0; c < dk; ++c) {
                    qt[c] *= iq;
                    kt[c] *= ik;
                }
            }
            /* channel-wise forget gate: alpha = exp(g), g in (lb, 0) */
            for (int64_t c = 0; c < dk; ++c) {
                const double a = gate[(t * H + h) * dk + c];
                const double g = gate_is_log ? fmax(a, gate_lower_bound)
                                             : gate_lower_bound * sigmoid(a);
                alpha[c] = exp(g);
            }
            const double b = beta[t * H + h];
            /* decay the rows of S, then the delta error against the decayed state */
            for (int64_t j = 0; j < dv; ++j)
                u[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                double *row = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) {
                    row[j] *= alpha[i];
                    u[j] += row[j] * kt[i];
                }
            }
            for (int64_t j = 0; j < dv; ++j)
                u[j] = b * (vt[j] - u[j]);
            /* write along k, then the query reads the updated state */
            for (int64_t j = 0; j < dv; ++j)
                ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                double *row = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) {
                    row[j] += kt[i] * u[j];
                    ot[j] += row[j] * qt[i];
                }
            }
            for (int64_t j = 0; j < dv; ++j)
                o[(t * H + h) * dv + j] = scale * ot[j];
        }

        if (state_out)
            memcpy(state_out + pr * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
        free(qt);
        free(kt);
        free(vt);
        free(alpha);
        free(u);
        free(ot);
    }

    /* conv state: last three raw tokens; done after every head has read the
     * input state, since the output may alias it */
    if (conv_state_out) {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)(num_seqs * 3 * CC));
        for (int64_t n = 0; n < num_seqs; ++n) {
            const int64_t s0 = cu_seqlens[n], L = cu_seqlens[n + 1] - cu_seqlens[n];
            for (int s = 0; s < 3; ++s) {
                double *dst = tmp + (n * 3 + s) * CC;
                for (int64_t c = 0; c < H * dk; ++c) {
                    dst[c] = tail_value(q, H * dk, c, s0, L, s, conv_state_in, CC, n, c);
                    dst[H * dk + c] = tail_value(k, H * dk, c, s0, L, s, conv_state_in,
                                                 CC, n, H * dk + c);
                }
                for (int64_t c = 0; c < H * dv; ++c)
                    dst[2 * H * dk + c] = tail_value(v, H * dv, c, s0, L, s, conv_state_in,
                                                     CC, n, 2 * H * dk + c);
            }
        }
        memcpy(conv_state_out, tmp, sizeof(double) * (size_t)(num_seqs * 3 * CC));
        free(tmp);
    }
}

/*
 * One decode step: every sequence receives one token.  It is the same
 * recurrence for a sequence of length one, continuing from the given state
 * and conv cache, both updated in place.
 *   q, k, gate : [num_seqs][H][dk];  v, o : [num_seqs][H][dv];  beta [num_seqs][H]
 *   conv_state : [num_seqs][3][2*H*dk + H*dv];  state : [num_seqs][H][dk][dv]
 */
void kda_oracle_decode(int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                       const double *q, const double *k, const double *v,
                       const double *gate, const double *beta,
                       const double *conv_w, const double *conv_b,
                       double *conv_state, double *state, double *o,
                       double scale, double gate_lower_bound, unsigned flags,
                       int nthreads)
{
    int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(num_seqs + 1));
    for (int64_t n = 0; n <= num_seqs; ++n)
        cu[n] = (int32_t)n;
    kda_oracle_prefill(num_seqs, H, dk, dv, cu, q, k, v, gate, beta, conv_w, conv_b,
                       conv_state, conv_state, state, state, o, scale,
                       gate_lower_bound, flags, nthreads);
    free(cu);
}
