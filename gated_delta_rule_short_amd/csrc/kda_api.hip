// kda_api.hip -- the extern "C" entry points of libkda.so (declared in kda.h).
//
// Every argument is checked on the host before anything is enqueued; failures
// return a status code and leave a message in a thread-local buffer.  The
// library allocates nothing and never synchronises the stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kda_status hip_fail(hipError_t e, const char *what) {
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t esize(kda_dtype d) { return d == KDA_BF16 ? 2 : 4; }
size_t state_esize(uint32_t flags) { return (flags & KDA_F_STATE_BF16) ? 2 : 4; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

// Checks an optional host copy of cu_seqlens.
kda_status check_cu_host(const int32_t *cu, int32_t n, int64_t total) {
    if (!cu) return KDA_OK;
    if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int32_t i = 0; i < n; ++i)
        if (cu[i + 1] < cu[i])
            return fail(KDA_ERR_INVALID_ARG, "cu_seqlens not monotone at %d (%d > %d)", i, cu[i],
                        cu[i + 1]);
    if ((int64_t)cu[n] != total)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[%d] = %d, expected total_tokens = %lld", n,
                    cu[n], (long long)total);
    return KDA_OK;
}

kda_status check_common(int32_t num_seqs, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                        uint32_t flags, float scale, float lb, uint32_t allowed = KDA_F_ALL) {
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs = %d, must be >= 1", num_seqs);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "num_heads = %d, must be >= 1", H);
    if (dk != 128 || dv != 128)
        return fail(KDA_ERR_UNSUPPORTED, "head dims %d x %d: only 128 x 128 is supported", dk, dv);
    if (dt != KDA_F32 && dt != KDA_BF16) return fail(KDA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
    if (flags & ~allowed) return fail(KDA_ERR_UNSUPPORTED, "unsupported flags 0x%x", flags);
    if (!std::isfinite(scale) || scale < 0.f)
        return fail(KDA_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 = default)");
    if (!std::isfinite(lb) || !(lb < 0.f))
        return fail(KDA_ERR_INVALID_ARG, "gate_lower_bound must be finite and < 0");
    if ((int64_t)num_seqs * H > (int64_t)1 << 26)
        return fail(KDA_ERR_INVALID_ARG, "num_seqs * num_heads too large");
    return KDA_OK;
}

// Rows of the state and conv-state arrays: the pool size with a slot map, else
// one per sequence.
kda_status pool_rows(const int32_t *slots, int32_t num_slots, int32_t num_seqs, size_t &rows) {
    if (!slots) {
        rows = (size_t)num_seqs;
        return KDA_OK;
    }
    if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "state_slots needs num_slots >= 1");
    rows = (size_t)num_slots;
    return KDA_OK;
}

int env_int(const char *name, int dflt) {
    const char *v = std::getenv(name);
    return v && *v ? std::atoi(v) : dflt;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(int s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        default: return "KDA_UNKNOWN_STATUS";
    }
}

const char *kda_last_error(void) { return g_err; }

kda_status kda_short_conv(const void *x, void *y, int64_t total_tokens, int32_t channels,
                          const float *weight, const float *bias, const void *conv_state_in,
                          void *conv_state_out, const int32_t *cu_seqlens,
                          const int32_t *cu_seqlens_host, int32_t num_seqs, kda_dtype dtype,
                          uint32_t flags, hipStream_t stream) {
    g_err[0] = 0;
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs = %d, must be >= 1", num_seqs);
    if (channels < 1) return fail(KDA_ERR_INVALID_ARG, "channels = %d, must be >= 1", channels);
    if (total_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens < 0");
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (flags & ~(uint32_t)KDA_F_SILU)
        return fail(KDA_ERR_UNSUPPORTED, "kda_short_conv accepts only KDA_F_SILU (flags 0x%x)", flags);
    if (!weight) return fail(KDA_ERR_INVALID_ARG, "weight is NULL");
    if (total_tokens > 0 && (!x || !y)) return fail(KDA_ERR_INVALID_ARG, "x or y is NULL");
    if (!cu_seqlens && total_tokens % num_seqs)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens NULL needs total_tokens %% num_seqs == 0");
    if (cu_seqlens && cu_seqlens_host == nullptr && num_seqs < 1)
        return fail(KDA_ERR_INVALID_ARG, "bad cu_seqlens");
    kda_status st = check_cu_host(cu_seqlens_host, num_seqs, total_tokens);
    if (st != KDA_OK) return st;
    const size_t bytes = (size_t)total_tokens * channels * esize(dtype);
    if (overlap(x, bytes, y, bytes)) return fail(KDA_ERR_INVALID_ARG, "y overlaps x");
    const size_t csb = (size_t)num_seqs * 3 * channels * esize(dtype);
    if (conv_state_out && conv_state_out != conv_state_in &&
        overlap(conv_state_out, csb, conv_state_in, csb))
        return fail(KDA_ERR_INVALID_ARG, "conv_state_out partially overlaps conv_state_in");
    if (total_tokens > 0) {
        hipError_t e = kda::launch_short_conv(dtype, x, y, total_tokens, channels, weight, bias,
                                              conv_state_in, cu_seqlens, num_seqs,
                                              (flags & KDA_F_SILU) != 0, stream);
        if (e != hipSuccess) return hip_fail(e, "short_conv launch");
    }
    if (conv_state_out) {
        const void *src[3] = {x, x, x};
        const int ch[3] = {channels, 0, 0};
        hipError_t e = kda::launch_conv_tail(dtype, src, ch, total_tokens, conv_state_in,
                                             conv_state_out, cu_seqlens, num_seqs, nullptr, 0,
                                             stream);
        if (e != hipSuccess) return hip_fail(e, "conv tail launch");
    }
    return KDA_OK;
}

size_t kda_prefill_workspace_size(const kda_prefill_args *a) {
    if (!a || a->dtype != KDA_BF16 || (a->chunk_size != 0 && a->chunk_size != 16)) return 0;
    if (a->num_seqs < 1 || a->num_heads < 1 || a->total_tokens < 0) return 0;
    return kda::split_workspace_bytes(a->total_tokens, a->num_seqs, a->num_heads);
}

kda_status kda_prefill(const kda_prefill_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    kda_status st = check_common(a->num_seqs, a->num_heads, a->head_dim_k, a->head_dim_v, a->dtype,
                                 a->flags, a->scale, a->gate_lower_bound);
    if (st != KDA_OK) return st;
    if (a->total_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens < 0");
    // token positions inside a sequence are 32-bit in the kernels (cu_seqlens is int32)
    if (a->total_tokens > ((int64_t)1 << 31) - 64) return fail(KDA_ERR_INVALID_ARG, "total_tokens too large");
    int chunk = a->chunk_size;
    if (chunk == 0) chunk = a->dtype == KDA_BF16 ? 64 : 32;
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: use 16, 32 or 64", a->chunk_size);
    if (a->dtype == KDA_F32 && chunk == 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size 64 needs bf16 I/O (fp32 staging exceeds LDS)");
    if (!a->conv_weight) return fail(KDA_ERR_INVALID_ARG, "conv_weight is NULL");
    if (a->total_tokens > 0 &&
        (!a->q || !a->k || !a->v || !a->gate || !a->beta || !a->o))
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, gate, beta and o must be non-NULL");
    if (!a->cu_seqlens && a->total_tokens % a->num_seqs)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens NULL needs total_tokens %% num_seqs == 0");
    st = check_cu_host(a->cu_seqlens_host, a->num_seqs, a->total_tokens);
    if (st != KDA_OK) return st;
    const int64_t T = a->total_tokens, H = a->num_heads;
    const size_t es = esize(a->dtype);
    const size_t tok = (size_t)T * H * 128 * es;
    const void *ins[4] = {a->q, a->k, a->v, a->gate};
    for (const void *in : ins)
        if (overlap(a->o, tok, in, tok)) return fail(KDA_ERR_INVALID_ARG, "o overlaps an input");
    if (overlap(a->o, tok, a->beta, (size_t)T * H * es))
        return fail(KDA_ERR_INVALID_ARG, "o overlaps beta");
    size_t rows = 0;
    st = pool_rows(a->state_slots, a->num_slots, a->num_seqs, rows);
    if (st != KDA_OK) return st;
    const size_t sb = rows * H * 128 * 128 * state_esize(a->flags);
    if (a->state_out && (const void *)a->state_out != (const void *)a->state_in &&
        overlap(a->state_out, sb, a->state_in, sb))
        return fail(KDA_ERR_INVALID_ARG, "state_out partially overlaps state_in");
    if (overlap(a->state_out, sb, a->o, tok)) return fail(KDA_ERR_INVALID_ARG, "state_out overlaps o");
    const size_t csb = rows * 3 * 3 * H * 128 * es;
    if (a->conv_state_out && a->conv_state_out != a->conv_state_in &&
        overlap(a->conv_state_out, csb, a->conv_state_in, csb))
        return fail(KDA_ERR_INVALID_ARG, "conv_state_out partially overlaps conv_state_in");

    kda_prefill_args args = *a;
    if (args.scale == 0.f) args.scale = 1.0f / std::sqrt(128.0f);
    const int64_t pairs = (int64_t)a->num_seqs * H;
    const size_t need = kda_prefill_workspace_size(a);
    const bool two_pass = need > 0 && a->workspace && a->workspace_bytes >= need;
    if (two_pass) {
        const size_t wb = a->workspace_bytes;
        if (overlap(a->workspace, wb, a->o, tok) || overlap(a->workspace, wb, a->state_out, sb))
            return fail(KDA_ERR_INVALID_ARG, "workspace overlaps an output");
        for (const void *in : ins)
            if (overlap(a->workspace, wb, in, tok))
                return fail(KDA_ERR_INVALID_ARG, "workspace overlaps an input");
    }
    // dv tile per workgroup: enough workgroups for 256 compute units.  The tile
    // changes only which workgroup computes a column, not the arithmetic.
    int dv_tile = pairs >= 256 ? 128 : (pairs >= 128 ? 64 : 32);
    const int forced = env_int("KDA_PREFILL_DV_TILE", 0);
    if (forced == 32 || forced == 64 || forced == 128 || (two_pass && forced == 16)) dv_tile = forced;
    hipError_t e;
    if (two_pass) {
        e = kda::launch_prefill_split(&args, dv_tile, stream);
    } else {
        kda::PrefillLaunch pl{&args, chunk, dv_tile};
        e = kda::launch_prefill(pl, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    if (a->conv_state_out) {
        const void *src[3] = {a->q, a->k, a->v};
        const int c = (int)(H * 128);
        const int ch[3] = {c, c, c};
        e = kda::launch_conv_tail(a->dtype, src, ch, T, a->conv_state_in, a->conv_state_out,
                                  a->cu_seqlens, a->num_seqs, a->state_slots, a->num_slots,
                                  stream);
        if (e != hipSuccess) return hip_fail(e, "conv tail launch");
    }
    return KDA_OK;
}

kda_status kda_decode(const kda_decode_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    kda_status st = check_common(a->num_seqs, a->num_heads, a->head_dim_k, a->head_dim_v, a->dtype,
                                 a->flags, a->scale, a->gate_lower_bound);
    if (st != KDA_OK) return st;
    if (!a->q || !a->k || !a->v || !a->gate || !a->beta || !a->o || !a->conv_weight ||
        !a->conv_state || !a->state)
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, gate, beta, o, conv_weight, conv_state and "
                                         "state must be non-NULL");
    const size_t es = esize(a->dtype);
    const size_t tok = (size_t)a->num_seqs * a->num_heads * 128 * es;
    size_t rows = 0;
    st = pool_rows(a->state_slots, a->num_slots, a->num_seqs, rows);
    if (st != KDA_OK) return st;
    const size_t sb = rows * a->num_heads * 128 * 128 * state_esize(a->flags);
    const size_t cb = rows * 3 * 3 * a->num_heads * 128 * es;
    const void *ins[4] = {a->q, a->k, a->v, a->gate};
    for (const void *in : ins) {
        if (overlap(a->o, tok, in, tok)) return fail(KDA_ERR_INVALID_ARG, "o overlaps an input");
        if (overlap(a->state, sb, in, tok)) return fail(KDA_ERR_INVALID_ARG, "state overlaps an input");
    }
    if (overlap(a->state, sb, a->o, tok)) return fail(KDA_ERR_INVALID_ARG, "state overlaps o");
    if (overlap(a->state, sb, a->conv_state, cb) || overlap(a->conv_state, cb, a->o, tok))
        return fail(KDA_ERR_INVALID_ARG, "conv_state overlaps state or o");
    kda_decode_args args = *a;
    if (args.scale == 0.f) args.scale = 1.0f / std::sqrt(128.0f);
    hipError_t e = kda::launch_decode(&args, stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return KDA_OK;
}

kda_status kda_decode_multi(const kda_decode_multi_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    kda_status st = check_common(a->num_seqs, a->num_heads, a->head_dim_k, a->head_dim_v, a->dtype,
                                 a->flags, a->scale, a->gate_lower_bound);
    if (st != KDA_OK) return st;
    if (a->num_tokens < 1 || a->num_tokens > KDA_MAX_SPEC_TOKENS)
        return fail(KDA_ERR_INVALID_ARG, "num_tokens = %d, must be in 1..%d", a->num_tokens,
                    KDA_MAX_SPEC_TOKENS);
    if (!a->q || !a->k || !a->v || !a->gate || !a->beta || !a->o || !a->conv_weight ||
        !a->conv_state || !a->state || !a->updates)
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, gate, beta, o, conv_weight, conv_state, state "
                                         "and updates must be non-NULL");
    if (a->pending_updates) {
        if (!a->pending_accepted)
            return fail(KDA_ERR_INVALID_ARG, "pending_updates needs pending_accepted");
        if (a->pending_tokens < 1 || a->pending_tokens > KDA_MAX_SPEC_TOKENS)
            return fail(KDA_ERR_INVALID_ARG, "pending_tokens = %d, must be in 1..%d",
                        a->pending_tokens, KDA_MAX_SPEC_TOKENS);
    }
    const size_t es = esize(a->dtype);
    const size_t NH = (size_t)a->num_seqs * a->num_heads;
    const size_t tok = NH * a->num_tokens * 128 * es;
    size_t rows = 0;
    st = pool_rows(a->state_slots, a->num_slots, a->num_seqs, rows);
    if (st != KDA_OK) return st;
    const size_t sb = rows * a->num_heads * 128 * 128 * state_esize(a->flags);
    const size_t cb = rows * 3 * 3 * a->num_heads * 128 * es;
    const size_t rb = NH * a->num_tokens * KDA_UPDATE_FLOATS * 4;
    const size_t pb = a->pending_updates ? NH * a->pending_tokens * KDA_UPDATE_FLOATS * 4 : 0;
    const void *ins[4] = {a->q, a->k, a->v, a->gate};
    for (const void *in : ins) {
        if (overlap(a->o, tok, in, tok)) return fail(KDA_ERR_INVALID_ARG, "o overlaps an input");
        if (overlap(a->updates, rb, in, tok))
            return fail(KDA_ERR_INVALID_ARG, "updates overlaps an input");
        if (overlap(a->state, sb, in, tok) || overlap(a->conv_state, cb, in, tok))
            return fail(KDA_ERR_INVALID_ARG, "state or conv_state overlaps an input");
    }
    if (overlap(a->state, sb, a->o, tok) || overlap(a->conv_state, cb, a->o, tok))
        return fail(KDA_ERR_INVALID_ARG, "state or conv_state overlaps o");
    if (overlap(a->updates, rb, a->o, tok) || overlap(a->updates, rb, a->state, sb) ||
        overlap(a->updates, rb, a->conv_state, cb))
        return fail(KDA_ERR_INVALID_ARG, "updates overlaps o, state or conv_state");
    if (overlap(a->updates, rb, a->pending_updates, pb))
        return fail(KDA_ERR_INVALID_ARG, "updates overlaps pending_updates");
    if (overlap(a->pending_updates, pb, a->state, sb) ||
        overlap(a->pending_updates, pb, a->conv_state, cb))
        return fail(KDA_ERR_INVALID_ARG, "pending_updates overlaps state or conv_state");
    kda_decode_multi_args args = *a;
    if (args.scale == 0.f) args.scale = 1.0f / std::sqrt(128.0f);
    hipError_t e = kda::launch_decode_multi(&args, stream);
    if (e != hipSuccess) return hip_fail(e, "decode_multi launch");
    return KDA_OK;
}

kda_status kda_decode_commit(const kda_decode_commit_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    kda_status st = check_common(a->num_seqs, a->num_heads, a->head_dim_k, a->head_dim_v, a->dtype,
                                 a->flags, 0.f, -1.f, KDA_F_STATE_BF16);
    if (st != KDA_OK) return st;
    if (a->num_tokens < 1 || a->num_tokens > KDA_MAX_SPEC_TOKENS)
        return fail(KDA_ERR_INVALID_ARG, "num_tokens = %d, must be in 1..%d", a->num_tokens,
                    KDA_MAX_SPEC_TOKENS);
    if (!a->accepted || !a->updates || !a->conv_state || !a->state)
        return fail(KDA_ERR_INVALID_ARG, "accepted, updates, conv_state and state must be non-NULL");
    const size_t NH = (size_t)a->num_seqs * a->num_heads;
    size_t rows = 0;
    st = pool_rows(a->state_slots, a->num_slots, a->num_seqs, rows);
    if (st != KDA_OK) return st;
    const size_t sb = rows * a->num_heads * 128 * 128 * state_esize(a->flags);
    const size_t cb = rows * 3 * 3 * a->num_heads * 128 * esize(a->dtype);
    const size_t rb = NH * a->num_tokens * KDA_UPDATE_FLOATS * 4;
    if (overlap(a->updates, rb, a->state, sb) || overlap(a->updates, rb, a->conv_state, cb) ||
        overlap(a->state, sb, a->conv_state, cb))
        return fail(KDA_ERR_INVALID_ARG, "updates, state and conv_state must not overlap");
    hipError_t e = kda::launch_decode_commit(a, stream);
    if (e != hipSuccess) return hip_fail(e, "decode_commit launch");
    return KDA_OK;
}

kda_status kda_state_copy(const kda_state_copy_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    if (a->count < 0) return fail(KDA_ERR_INVALID_ARG, "count = %d, must be >= 0", a->count);
    kda_status st = check_common(1, a->num_heads, a->head_dim_k, a->head_dim_v, a->dtype, a->flags,
                                 0.f, -1.f, KDA_F_STATE_BF16);
    if (st != KDA_OK) return st;
    if (a->num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1");
    if ((int64_t)a->num_slots * a->num_heads > (int64_t)1 << 26 ||
        (int64_t)a->count * a->num_heads > (int64_t)1 << 26)
        return fail(KDA_ERR_INVALID_ARG, "num_slots * num_heads or count * num_heads too large");
    if (!a->src_slots || !a->dst_slots || !a->state_src || !a->state_dst)
        return fail(KDA_ERR_INVALID_ARG, "src_slots, dst_slots, state_src and state_dst must be "
                                         "non-NULL");
    if (!a->conv_src != !a->conv_dst)
        return fail(KDA_ERR_INVALID_ARG, "conv_src and conv_dst must both be given or both NULL");
    const size_t sb = (size_t)a->num_slots * a->num_heads * 128 * 128 * state_esize(a->flags);
    const size_t cb = (size_t)a->num_slots * 3 * 3 * a->num_heads * 128 * esize(a->dtype);
    if (a->state_src != a->state_dst && overlap(a->state_src, sb, a->state_dst, sb))
        return fail(KDA_ERR_INVALID_ARG, "state_dst partially overlaps state_src");
    if (a->conv_src != a->conv_dst && overlap(a->conv_src, cb, a->conv_dst, cb))
        return fail(KDA_ERR_INVALID_ARG, "conv_dst partially overlaps conv_src");
    if (overlap(a->state_dst, sb, a->conv_src, cb) || overlap(a->state_dst, sb, a->conv_dst, cb) ||
        overlap(a->conv_dst, cb, a->state_src, sb))
        return fail(KDA_ERR_INVALID_ARG, "state and conv-state pools overlap");
    if (a->count == 0) return KDA_OK;
    hipError_t e = kda::launch_state_copy(a, stream);
    if (e != hipSuccess) return hip_fail(e, "state_copy launch");
    return KDA_OK;
}

size_t kda_gate_beta_workspace_size(const kda_gate_beta_args *a) {
    if (!a || a->total_tokens < 0 || a->num_heads < 1) return 0;
    return kda::gate_proj_workspace_bytes(a->total_tokens, a->num_heads);
}

kda_status kda_gate_beta_proj(const kda_gate_beta_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    const int64_t T = a->total_tokens;
    if (T < 0) return fail(KDA_ERR_INVALID_ARG, "total_tokens < 0");
    if (T > ((int64_t)1 << 31) - 64) return fail(KDA_ERR_INVALID_ARG, "total_tokens too large");
    if (a->hidden < 256 || a->hidden % 256)  // four K quarters of whole 64-wide super-steps
        return fail(KDA_ERR_UNSUPPORTED, "hidden = %d: a positive multiple of 256 is needed", a->hidden);
    if (a->rank != 128) return fail(KDA_ERR_UNSUPPORTED, "rank = %d: only 128 is supported", a->rank);
    if (a->head_dim_k != 128)
        return fail(KDA_ERR_UNSUPPORTED, "head_dim_k = %d: only 128 is supported", a->head_dim_k);
    if (a->num_heads != 64 && a->num_heads != 128)
        return fail(KDA_ERR_UNSUPPORTED, "num_heads = %d: 64 or 128", a->num_heads);
    // (H * 128 gate channels: a multiple of the 1024 channels of an expansion workgroup)
    if (a->flags & ~(uint32_t)KDA_F_GATE_IS_LOG)
        return fail(KDA_ERR_UNSUPPORTED, "unsupported flags 0x%x", a->flags);
    if (!std::isfinite(a->gate_lower_bound) || !(a->gate_lower_bound < 0.f))
        return fail(KDA_ERR_INVALID_ARG, "gate_lower_bound must be finite and < 0");
    if (T == 0) return KDA_OK;
    const void *ptrs[8] = {a->x, a->w_a, a->w_b, a->w_beta, a->gate, a->beta, a->workspace, nullptr};
    for (int i = 0; i < 7; ++i) {
        if (!ptrs[i])
            return fail(KDA_ERR_INVALID_ARG, "x, w_a, w_b, w_beta, gate, beta and workspace must be "
                                             "non-NULL");
        if ((uintptr_t)ptrs[i] % 16)
            return fail(KDA_ERR_INVALID_ARG, "every tensor must be 16-byte aligned");
    }
    const size_t need = kda::gate_proj_workspace_bytes(T, a->num_heads);
    if (a->workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", a->workspace_bytes, need);
    const size_t H = (size_t)a->num_heads, hid = (size_t)a->hidden;
    const size_t xb = (size_t)T * hid * 2, gb = (size_t)T * H * 128 * 2, bb = (size_t)T * H * 2;
    const void *ins[4] = {a->x, a->w_a, a->w_b, a->w_beta};
    const size_t inb[4] = {xb, 128 * hid * 2, H * 128 * 128 * 2, H * hid * 2};
    const void *outs[3] = {a->gate, a->beta, a->workspace};
    const size_t outb[3] = {gb, bb, need};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[o], outb[o], ins[i], inb[i]))
                return fail(KDA_ERR_INVALID_ARG, "an output or the workspace overlaps an input");
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (overlap(outs[o], outb[o], outs[o2], outb[o2]))
                return fail(KDA_ERR_INVALID_ARG, "gate, beta and workspace must not overlap");
    }
    hipError_t e = kda::launch_gate_proj(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gate_beta_proj launch");
    return KDA_OK;
}

}  // extern "C"
