/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) implementation of the
 * Kimi Delta Attention (KDA) sequence mixer.
 *
 * The operation (source: "GLM-5.3-Flash im Detail" (flozi.net), section
 * "Sequenz-Mixing: 34 KDA-Schichten mit festem Zustand"; the dataset card
 * "GLM-5.3-Flash Internals", section "Anatomy", gives the same shape):
 * per head (64 heads of dimension 128 in the published model) q, k and v pass
 * through a causal depthwise convolution of width 4; a channel-wise forget gate
 * with log-decay bounded below at -5 attenuates a matrix state; a scalar beta
 * drives a delta-rule write of v along k; the query reads the updated state.
 * Prefill evaluates tokens inside chunks in parallel and passes a state between
 * chunks; decode of one token is a recurrent update (same section).  The state
 * is a dk x dv matrix per head held in fp32 (same section, the state-size
 * arithmetic), and prefill and decode share one state layout (same page,
 * section "FP8-Checkpoint und Betriebsgrenzen": identical KDA layouts when
 * prefill and decode run separately).
 *
 * Per token t of a sequence and per head, with conv-ed, L2-normalised q_t, k_t:
 *     S   <- diag(exp(g_t)) S                 g_t = lb * sigmoid(a_t), lb = -5
 *     u   =  beta_t * (v_t - S^T k_t)
 *     S   <- S + k_t u^T
 *     o_t =  scale * S^T q_t
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer.  The library never allocates,
 *     frees or synchronises; work is enqueued asynchronously on `stream`.
 *   - Pointers: all tensor pointers are DEVICE pointers, except the optional
 *     `cu_seqlens_host`, which is a HOST pointer used only for validation.
 *   - Layouts are dense row-major with the last index fastest.  T = total
 *     tokens of all packed sequences, N = number of sequences, H = heads,
 *     dk = dv = 128, CC = 2*H*dk + H*dv conv channels ordered q, k, v
 *     (head-major, channel fastest inside each).
 *   - dtype (kda_dtype) applies to q, k, v, gate, beta, o and conv states;
 *     conv weights/biases and the recurrent state are always fp32.
 *   - Errors: every argument check runs on the host before any launch and
 *     returns KDA_ERR_INVALID_ARG (bad pointer, size, layout) or
 *     KDA_ERR_UNSUPPORTED (head dim != 128, unknown flag, unsupported chunk).
 *     A failed launch returns KDA_ERR_HIP.  kda_last_error() gives a message
 *     for the calling thread's last failure.  No exception crosses the ABI.
 *   - Thread safety: no global mutable state besides that per-thread message
 *     (and kda_prefill_noalloc's per-GPU scratch, see there); concurrent calls
 *     on different buffers are safe.
 *
 * State pool (prefill, decode, decode_multi, decode_commit).  By default
 * sequence n of a call owns row n of the state and conv-state arrays.  With
 * `state_slots` (int32 [N], device memory) it owns row state_slots[n] of a pool
 * of `num_slots` rows instead: the state and conv-state arguments then point
 * to [num_slots][...] arrays, and a serving loop keeps every live sequence's
 * state resident and passes each call's batch as slot numbers.  Prefix reuse
 * fits the same pool: kda_state_copy snapshots or forks slots.  The disaggregated
 * deployment of the pages keeps identical KDA layouts for prefill and decode
 * ("GLM-5.3-Flash im Detail", section "FP8-Checkpoint und Betriebsgrenzen"),
 * and this pool is one such layout.  Slots of one call must be distinct.  A
 * slot outside [0, num_slots) cannot be checked on the host; on the device
 * that sequence is skipped: none of its outputs, state or conv state is read
 * or written.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 6

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,
    KDA_ERR_UNSUPPORTED = 2,
    KDA_ERR_HIP = 3,
    KDA_STATUS_INT_RANGE = 0x7fffffff  /* never returned: makes every int a valid kda_status
                                          value, so kda_status_string may be given any int */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Flags.  The pages do not say whether an activation follows the conv, whether
 * q/k are L2-normalised, or how the gate is parameterised; these flags select
 * the alternatives (default: no activation, L2 on, g = lb * sigmoid(a)). */
enum {
    KDA_F_SILU = 1u,          /* y <- y * sigmoid(y) after the conv (q, k and v) */
    KDA_F_NO_QK_L2NORM = 2u,  /* skip q/k L2 normalisation x / sqrt(|x|^2 + 1e-6) */
    KDA_F_GATE_IS_LOG = 4u,   /* gate holds the log-decay: g = max(gate, lb) */
    KDA_F_STATE_BF16 = 8u     /* the recurrent state is stored as bf16 (see below) */
};
#define KDA_F_ALL (KDA_F_SILU | KDA_F_NO_QK_L2NORM | KDA_F_GATE_IS_LOG | KDA_F_STATE_BF16)

/* 16-bit state storage (KDA_F_STATE_BF16).  One page prints the 1M-context
 * state as 0.07 GB, which is the 64x128x128 per layer and 34 layers at 2 bytes
 * per value, while the state-size arithmetic of the same source stores FP32
 * ("GLM-5.3-Flash im Detail", section "Sequenz-Mixing" and the KV-cache
 * derivation).  With the flag, kda_prefill (state_in, state_out), kda_decode,
 * kda_decode_multi and kda_decode_commit read and write the state as bf16
 * [N][H][dk][dv]: each call widens it exactly to fp32, runs the same fp32
 * arithmetic, and rounds the result to nearest even once when it stores it.
 * It halves the state traffic, the whole cost of a decode step.  Rounding once
 * per call adds error that levels off rather than growing with the number of
 * steps, at a size set by how slowly the state decays; fp32 stays the
 * default.  Supported regime: measured against the fp64 recurrence over 256 to
 * 8192 decode steps, outputs and states stay within a relative error of 2e-2
 * while the per-row decays exp(g) stay below about 0.998 (memories of up to
 * about 600 tokens); with decays near 0.9998 the error levels off at about
 * 2.4e-2.  Keep fp32 storage where the gates hold the state that long. */

/* Version of this ABI (KDA_ABI_VERSION). */
int kda_abi_version(void);

/*
 * Bound of the fused prefill's hand-over waits (KDA_SCHEDULE_FUSED), for tests of
 * its failure path.  A wave of the fused kernel waits for a ring slot or a record
 * by polling a word in LDS; after `polls` unsuccessful polls it gives up and
 * marks the workgroup, whose waves then wait no more: the call still ends, with
 * wrong results, instead of hanging.  The default (2^22 polls, restored by any
 * polls <= 0) is never reached by a correct hand-over.  Process-wide; takes
 * effect for launches after the call; returns the previous bound.
 */
int32_t kda_set_spin_limit(int32_t polls);

/* Static string naming a kda_status value ("KDA_UNKNOWN_STATUS" for any other value). */
const char *kda_status_string(kda_status status);

/* Message describing the calling thread's most recent failing call ("" if none). */
const char *kda_last_error(void);

/*
 * kda_short_conv -- causal depthwise convolution of width 4 over packed
 * sequences (the conv step of the passage above, on its own).
 *   x, y            [T][channels] in `dtype`; y must not overlap x.
 *   weight          [channels][4] fp32; tap 3 multiplies the current token,
 *                   taps 0..2 the three previous tokens of the same sequence.
 *   bias            [channels] fp32 or NULL.
 *   conv_state_in   [N][3][channels] or NULL (zeros): the three raw tokens
 *                   before each sequence, oldest first.
 *   conv_state_out  [N][3][channels] or NULL: the last three raw tokens of
 *                   (conv_state_in ++ sequence); may alias conv_state_in.
 *   cu_seqlens      [N+1] int32 device prefix sums (cu[0] = 0, cu[N] = T), or
 *                   NULL for N equal sequences of T/N tokens.
 *   cu_seqlens_host optional host copy of cu_seqlens; when given it is
 *                   checked (monotone, cu[0] = 0, cu[N] = T).
 *   flags           0 or KDA_F_SILU.
 * A sequence never reads another sequence's tokens.  Empty sequences are
 * allowed (their conv state passes through).
 */
kda_status kda_short_conv(const void *x, void *y, int64_t total_tokens, int32_t channels,
                          const float *weight, const float *bias,
                          const void *conv_state_in, void *conv_state_out,
                          const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                          int32_t num_seqs, kda_dtype dtype, uint32_t flags,
                          hipStream_t stream);

/*
 * kda_prefill -- chunk-parallel prefill of packed sequences (the prefill
 * kernel shape of the passage above): tokens inside a chunk are evaluated in
 * parallel through the WY/UT form, the fp32 state is carried from chunk to
 * chunk.
 */
typedef struct {
    int32_t num_seqs;        /* N >= 1 */
    int32_t num_heads;       /* H >= 1 */
    int32_t head_dim_k;      /* must be 128 */
    int32_t head_dim_v;      /* must be 128 */
    int32_t chunk_size;      /* 0 = default; 16, 32 or 64.  The fused and two-pass
                                schedules use 16-token sub-chunks (0 or 16); the
                                one-pass default is 64-token chunks for bf16 and
                                32-token chunks for fp32 I/O (an fp32 64-token
                                chunk does not fit in LDS: KDA_ERR_UNSUPPORTED) */
    int64_t total_tokens;    /* 0 <= T <= 2^31 - 64 (token offsets are int32) */
    kda_dtype dtype;
    uint32_t flags;          /* KDA_F_* */
    float scale;             /* 0 = 1/sqrt(dk) */
    float gate_lower_bound;  /* lb of the log-decay, -5 in the published model; < 0 */
    const void *q, *k;       /* [T][H][dk] raw (pre-conv) */
    const void *v;           /* [T][H][dv] raw (pre-conv) */
    const void *gate;        /* [T][H][dk] pre-activation a (log-decay if GATE_IS_LOG) */
    const void *beta;        /* [T][H] write strength in [0, 1] */
    const float *conv_weight;/* [CC][4] */
    const float *conv_bias;  /* [CC] or NULL */
    const void *conv_state_in; /* [N][3][CC] or NULL (zeros) */
    void *conv_state_out;      /* [N][3][CC] or NULL; may alias conv_state_in */
    const void *state_in;      /* [N][H][dk][dv] fp32 (bf16 with KDA_F_STATE_BF16) or NULL */
    void *state_out;           /* [N][H][dk][dv], same type, or NULL; may alias state_in */
    void *o;                   /* [T][H][dv] output; must not overlap the inputs */
    const int32_t *cu_seqlens; /* [N+1] device, or NULL for N equal sequences */
    const int32_t *cu_seqlens_host; /* optional host copy, validated when given */
    void *workspace;           /* device scratch for the two-pass schedule, or NULL */
    size_t workspace_bytes;    /* its size; see kda_prefill_workspace_size */
    const int32_t *state_slots;/* [N] device pool slots, or NULL (see "State pool") */
    int32_t num_slots;         /* pool rows when state_slots is given */
    int32_t dv_tile;           /* state columns per workgroup: 0 = chosen from the
                                  number of (sequence, head) pairs (and, for two
                                  passes, the host lengths); else 32, 64 or
                                  128 (and 16 for the two-pass schedule; the fused
                                  schedule takes 0 or 128).  Changes which
                                  workgroup computes a column, never the
                                  arithmetic: results are bit-identical. */
    int32_t schedule;          /* KDA_SCHEDULE_*; 0 = chosen (see below) */
} kda_prefill_args;

typedef enum {
    KDA_SCHEDULE_AUTO = 0,
    KDA_SCHEDULE_ONE_PASS = 1,
    KDA_SCHEDULE_TWO_PASS = 2,
    KDA_SCHEDULE_FUSED = 3,
} kda_schedule;

/* The automatic choice takes the fused schedule from this many (sequence, head)
 * pairs on (bf16 I/O, chunk_size 0 or 16): one and a half workgroups per compute
 * unit of the 256 of gfx950.  Below about that many the two-pass schedule, whose
 * first pass spreads over the whole GPU, was the faster one on ragged batches. */
#define KDA_FUSED_MIN_PAIRS 384

/*
 * Three schedules compute the same mixer (identical in exact arithmetic):
 *   - one pass (KDA_SCHEDULE_ONE_PASS): each workgroup owns a (sequence, head,
 *     dv tile) and runs the chunk's WY/UT transform itself (chunk_size 16, 32 or
 *     64; default 64); any dtype, no workspace;
 *   - two passes (KDA_SCHEDULE_TWO_PASS; bf16 I/O, chunk_size 0 or 16): a fully
 *     parallel pass turns every 16-token sub-chunk of every head into
 *     matrix-core operands in the workspace (13,824 bytes per sub-chunk and
 *     head), and a second pass carries the state over them.  It keeps the whole
 *     GPU busy when there are few (sequence, head) pairs;
 *   - fused (KDA_SCHEDULE_FUSED; bf16 I/O, chunk_size 0 or 16): one workgroup
 *     per (sequence, head) forms the same 16-token operands in its own LDS while
 *     it carries the state over them, so they never reach memory; no workspace.
 *     It needs enough pairs to fill the GPU (more than one workgroup per compute
 *     unit), and a pair's sub-chunks run one after another in its workgroup.
 * KDA_SCHEDULE_AUTO takes the fused schedule when it applies, there are at
 * least KDA_FUSED_MIN_PAIRS pairs and, when cu_seqlens_host is given, the
 * longest sequence holds at most 1.8 times the mean number of 16-token
 * sub-chunks per compute unit (num_heads x the sum over sequences of their
 * sub-chunks, over 256); else two passes when a workspace is given, else one
 * pass.  An explicit schedule that the dtype or chunk_size excludes
 * returns KDA_ERR_UNSUPPORTED; KDA_SCHEDULE_TWO_PASS without a workspace returns
 * KDA_ERR_INVALID_ARG.  The fused and one-pass schedules ignore the workspace.
 * Workspace and windows.  A workspace of kda_prefill_workspace_full_size()
 * bytes runs the whole call at once.  A smaller one, of at least
 * kda_prefill_workspace_min_size() bytes, runs it in windows: every sequence
 * advances by the same number of sub-chunks per window (as many as the
 * workspace holds next to an fp32 carry of every (sequence, head) state), so
 * the memory needed is bounded whatever the sequence lengths; results are bit
 * for bit those of the whole call.  kda_prefill_workspace_size() recommends the
 * whole-call size up to KDA_PREFILL_WORKSPACE_CAP bytes and windows beyond it.
 * Giving cu_seqlens_host lets the library count the windows exactly (without
 * it, it plans for one sequence holding every token, and windows past the
 * longest sequence do nothing).  A workspace below the minimum returns
 * KDA_ERR_INVALID_ARG.  The workspace is owned by the caller, overwritten by
 * each call, and must not be shared by concurrent calls.
 */
kda_status kda_prefill(const kda_prefill_args *args, hipStream_t stream);

/* Recommended workspace bytes for the two-pass schedule (whole call when that
 * fits in KDA_PREFILL_WORKSPACE_CAP, else windows within it); 0 when the call
 * will not run that schedule (fp32 I/O, an explicit chunk_size of 32 or 64, an
 * explicit one-pass or fused schedule, or the automatic choice of the fused
 * one).  Depends on num_seqs, num_heads, total_tokens, dtype, chunk_size,
 * schedule and cu_seqlens_host (the automatic schedule and the window count). */
#define KDA_PREFILL_WORKSPACE_CAP ((size_t)4 << 30)
size_t kda_prefill_workspace_size(const kda_prefill_args *args);

/* Two-pass workspace bytes for the whole call in one window (no cap); 0 when
 * the dtype or chunk_size excludes the two-pass schedule. */
size_t kda_prefill_workspace_full_size(const kda_prefill_args *args);

/* Smallest workspace the two-pass schedule accepts: one sub-chunk per sequence
 * per window plus the carry (or the whole call, if that is smaller); 0 when the
 * dtype or chunk_size excludes the schedule. */
size_t kda_prefill_workspace_min_size(const kda_prefill_args *args);

/*
 * kda_prefill_noalloc -- kda_prefill for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as kda_prefill, except that
 * `workspace` must be NULL and `workspace_bytes` 0 (else KDA_ERR_INVALID_ARG):
 * the two-pass schedule (bf16 I/O, chunk_size 0 or 16) runs in a scratch array
 * of KDA_PREFILL_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, in windows when the call needs more than that; the
 * fused and one-pass schedules need no scratch.  The schedule is chosen as for
 * kda_prefill, with the scratch array as the workspace.  The call allocates
 * nothing.  A call whose smallest two-pass workspace
 * (kda_prefill_workspace_min_size) exceeds the scratch returns
 * KDA_ERR_INVALID_ARG: use kda_prefill with a workspace for it.  Every call on
 * one GPU shares that GPU's scratch and leaves its contents behind (nothing in
 * it needs clearing between calls): calls that overlap in time on one GPU
 * (different streams or threads) race, and the caller must order them.
 */
#define KDA_PREFILL_SCRATCH_BYTES ((size_t)256 << 20)
kda_status kda_prefill_noalloc(const kda_prefill_args *args, hipStream_t stream);

/*
 * kda_decode -- one new token for each of N sequences (the single-token
 * recurrent update of the passage above).  The conv cache and the state are
 * updated in place; the state layout is the one kda_prefill writes.
 */
typedef struct {
    int32_t num_seqs;        /* N >= 1 */
    int32_t num_heads;       /* H >= 1 */
    int32_t head_dim_k;      /* must be 128 */
    int32_t head_dim_v;      /* must be 128 */
    kda_dtype dtype;
    uint32_t flags;          /* KDA_F_* (KDA_F_STATE_BF16 allowed) */
    float scale;             /* 0 = 1/sqrt(dk) */
    float gate_lower_bound;  /* < 0 */
    const void *q, *k;       /* [N][H][dk] raw */
    const void *v;           /* [N][H][dv] raw */
    const void *gate;        /* [N][H][dk] */
    const void *beta;        /* [N][H] */
    const float *conv_weight;/* [CC][4] */
    const float *conv_bias;  /* [CC] or NULL */
    void *conv_state;        /* [N][3][CC] in/out (shifted by one token) */
    void *state;             /* [N][H][dk][dv] in/out: fp32, or bf16 with KDA_F_STATE_BF16 */
    void *o;                 /* [N][H][dv] */
    const int32_t *state_slots; /* [N] device pool slots, or NULL (see "State pool") */
    int32_t num_slots;          /* pool rows when state_slots is given */
} kda_decode_args;

kda_status kda_decode(const kda_decode_args *args, hipStream_t stream);

/*
 * Speculative multi-token decode.  The serving rig of the pages runs a
 * one-layer draft head (MTP, k = 5 drafted tokens per step) whose proposals the
 * target model verifies, about four of five being accepted ("GLM-5.3-Flash
 * Internals", sections "Serve rig" and "Architecture" (MTP), and the research
 * directions on MTP acceptance; "GLM-5.3-Flash im Detail", the draft-path row of
 * the architecture table).  Verification feeds T = k + 1 tokens per sequence
 * through the mixer at once; only a prefix of them is kept, so the state may
 * advance over the accepted tokens only.
 *
 * kda_decode_multi evaluates T tokens per sequence in order, exactly as T calls
 * of kda_decode would (output t sees tokens 0..t-1 of the same call), but
 * leaves the state and the conv cache where they were and writes one update
 * record per (sequence, head, token) instead.  kda_decode_commit then advances
 * the state and conv cache over the first `accepted[n]` tokens of each sequence
 * from those records.  The same commit can be fused into the next
 * kda_decode_multi call (the `pending_*` fields), so that a steady-state
 * speculative step reads and writes each state once.  Given the same inputs,
 * the outputs and the committed state equal those of that many kda_decode calls
 * up to the order of fp32 additions (kda_decode spreads a state over more
 * threads and groups the 128-row column sums differently), and the conv cache
 * equals theirs exactly; a commit fused into the next kda_decode_multi call
 * equals a separate kda_decode_commit bit for bit.
 *
 * Update record of (sequence n, head h, token t): KDA_UPDATE_ROWS rows of 128
 * fp32 at updates + ((n * H + h) * T + t) * KDA_UPDATE_FLOATS:
 *   row 0  exp(g_t), the per-row decay of the state
 *   row 1  the conv-ed, normalised key k_t
 *   row 2  u_t = beta_t (v_t - S'^T k_t), the delta-rule value
 *   rows 3, 4, 5  the raw (pre-conv) q_t, k_t, v_t of head h, exact in fp32
 * so that the commit needs neither the token buffers nor the gates again.
 */
#define KDA_MAX_SPEC_TOKENS 8
#define KDA_UPDATE_ROWS 6
#define KDA_UPDATE_FLOATS (KDA_UPDATE_ROWS * 128)

typedef struct {
    int32_t num_seqs;        /* N >= 1 */
    int32_t num_heads;       /* H >= 1 */
    int32_t head_dim_k;      /* must be 128 */
    int32_t head_dim_v;      /* must be 128 */
    int32_t num_tokens;      /* T, 1..KDA_MAX_SPEC_TOKENS tokens per sequence */
    kda_dtype dtype;
    uint32_t flags;          /* KDA_F_* (KDA_F_STATE_BF16 allowed) */
    float scale;             /* 0 = 1/sqrt(dk) */
    float gate_lower_bound;  /* < 0 */
    const void *q, *k;       /* [N][T][H][dk] raw */
    const void *v;           /* [N][T][H][dv] raw */
    const void *gate;        /* [N][T][H][dk] */
    const void *beta;        /* [N][T][H] */
    const float *conv_weight;/* [CC][4] */
    const float *conv_bias;  /* [CC] or NULL */
    void *conv_state;        /* [N][3][CC]; written only by a pending commit */
    void *state;             /* [N][H][dk][dv] fp32 (bf16 with KDA_F_STATE_BF16);
                                written only by a pending commit */
    void *o;                 /* [N][T][H][dv] */
    float *updates;          /* [N][H][T][KDA_UPDATE_FLOATS] fp32 records (written) */
    /* Optional fused commit of the previous call, applied to state and conv_state
     * before the T new tokens are evaluated (NULL pending_updates: none). */
    const float *pending_updates;    /* that call's records; must not overlap updates */
    const int32_t *pending_accepted; /* [N] device: tokens of that call to keep */
    int32_t pending_tokens;          /* that call's T; the previous call must have had
                                        the same N, H and state_slots */
    const int32_t *state_slots; /* [N] device pool slots, or NULL (see "State pool") */
    int32_t num_slots;          /* pool rows when state_slots is given */
} kda_decode_multi_args;

kda_status kda_decode_multi(const kda_decode_multi_args *args, hipStream_t stream);

/*
 * kda_decode_commit -- advance state and conv cache over the first accepted[n]
 * tokens of sequence n, from the records one kda_decode_multi call wrote.
 * accepted[] lives in device memory (it is usually computed on the GPU); a
 * value outside [0, T] is clamped to that range, and 0 leaves the sequence
 * untouched.
 */
typedef struct {
    int32_t num_seqs;        /* N >= 1, as in the kda_decode_multi call */
    int32_t num_heads;       /* H >= 1 */
    int32_t head_dim_k;      /* must be 128 */
    int32_t head_dim_v;      /* must be 128 */
    int32_t num_tokens;      /* T of the kda_decode_multi call */
    kda_dtype dtype;         /* dtype of conv_state */
    uint32_t flags;          /* 0 or KDA_F_STATE_BF16 */
    const int32_t *accepted; /* [N] device */
    const float *updates;    /* [N][H][T][KDA_UPDATE_FLOATS] records */
    void *conv_state;        /* [N][3][CC] in/out */
    void *state;             /* [N][H][dk][dv] in/out, fp32 or bf16 */
    const int32_t *state_slots; /* [N] device pool slots, or NULL (see "State pool") */
    int32_t num_slots;          /* pool rows when state_slots is given */
} kda_decode_commit_args;

kda_status kda_decode_commit(const kda_decode_commit_args *args, hipStream_t stream);

/*
 * kda_state_copy -- copy `count` pool rows: state and conv state of slot
 * src_slots[i] to slot dst_slots[i] (a prefix snapshot, or a fork of a cached
 * prefix into a new sequence: the serving branch of "GLM-5.3-Flash Internals"
 * runs with prefix caching, see its context-ladder battery).  Source and destination pools may be the same
 * array.  A destination slot must not also be a source of the same call, and
 * destination slots must be distinct.  Pairs with a slot outside
 * [0, num_slots) are skipped on the device.
 */
typedef struct {
    int32_t count;           /* copies, >= 0 */
    int32_t num_heads;       /* H >= 1 */
    int32_t head_dim_k;      /* must be 128 */
    int32_t head_dim_v;      /* must be 128 */
    int32_t num_slots;       /* rows of each pool, >= 1 */
    kda_dtype dtype;         /* dtype of the conv states */
    uint32_t flags;          /* 0 or KDA_F_STATE_BF16 */
    const int32_t *src_slots;/* [count] device */
    const int32_t *dst_slots;/* [count] device */
    const void *state_src;   /* [num_slots][H][dk][dv] */
    void *state_dst;         /* [num_slots][H][dk][dv]; may be state_src */
    const void *conv_src;    /* [num_slots][3][CC], or NULL (state only) */
    void *conv_dst;          /* [num_slots][3][CC]; NULL exactly when conv_src is */
} kda_state_copy_args;

kda_status kda_state_copy(const kda_state_copy_args *args, hipStream_t stream);

/*
 * kda_gate_beta_proj -- the gate and beta in-projections that feed the mixer,
 * with their activations fused into the matrix-core epilogues.  The decoder
 * is 4096 wide and its activation batteries name a KDA gate projection and the
 * second factor ("g_b_proj") of a two-factor one ("GLM-5.3-Flash Internals",
 * sections "Anatomy" and the activation batteries); the gate is channel-wise with
 * log-decay >= lb and beta is one scalar per head and token ("GLM-5.3-Flash im
 * Detail", section "Sequenz-Mixing").  Per token x:
 *     a    = W_b (W_a x)              rank r = 128, H * dk channels head-major
 *     gate = a, or lb * sigmoid(a) with KDA_F_GATE_IS_LOG (then pass that flag
 *            to kda_prefill / kda_decode, which read it as the log-decay)
 *     beta = sigmoid(W_beta x)
 * The first product runs in bf16 with fp32 accumulation and is rounded to bf16
 * before the second.  All tensors are bf16 and 16-byte aligned; the workspace
 * is overwritten by each call and must not be shared by concurrent calls.
 */
typedef struct {
    int64_t total_tokens;    /* T >= 0 */
    int32_t hidden;          /* width of x: a positive multiple of 256 */
    int32_t rank;            /* r: must be 128 */
    int32_t num_heads;       /* H: 64 or 128 */
    int32_t head_dim_k;      /* must be 128 */
    uint32_t flags;          /* 0 or KDA_F_GATE_IS_LOG */
    float gate_lower_bound;  /* lb < 0 */
    const void *x;           /* [T][hidden] */
    const void *w_a;         /* [r][hidden] */
    const void *w_b;         /* [H * dk][r] */
    const void *w_beta;      /* [H][hidden] */
    void *gate;              /* [T][H][dk]: the mixer's gate input */
    void *beta;              /* [T][H] */
    void *workspace;         /* kda_gate_beta_workspace_size() bytes */
    size_t workspace_bytes;
} kda_gate_beta_args;

kda_status kda_gate_beta_proj(const kda_gate_beta_args *args, hipStream_t stream);

/* Workspace bytes kda_gate_beta_proj needs: 16 T (r + H) for the split first
 * product's fp32 partials, then 2 T r for z. */
size_t kda_gate_beta_workspace_size(const kda_gate_beta_args *args);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
