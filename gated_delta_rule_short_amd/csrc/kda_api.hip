// kda_api.hip -- the extern "C" entry points of libkda.so (declared in kda.h).
//
// Every argument is checked on the host before anything is enqueued; failures
// return a status code and leave a message in a thread-local buffer.  The
// library allocates nothing and never synchronises the stream.
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

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

// A call's buffers as (pointer, bytes, name); the first `n_written` are written
// by the call.  Every written buffer must overlap no other buffer of the call.
// NULL or empty buffers overlap nothing; an allowed in-place pair is passed with
// the input side's size set to 0.
struct Buf {
    const void *p;
    size_t bytes;
    const char *name;
};
kda_status check_written(const Buf *b, int n, int n_written) {
    for (int i = 0; i < n_written; ++i)
        for (int j = 0; j < n; ++j) {
            if (j == i || (j < n_written && j < i)) continue;
            if (overlap(b[i].p, b[i].bytes, b[j].p, b[j].bytes))
                return fail(KDA_ERR_INVALID_ARG, "%s overlaps %s", b[i].name, b[j].name);
        }
    return KDA_OK;
}

// The two-pass and fused schedules apply to bf16 I/O with chunk_size 0 or 16.
bool two_pass_applies(const kda_prefill_args *a) {
    return a && a->dtype == KDA_BF16 && (a->chunk_size == 0 || a->chunk_size == 16) && a->num_seqs >= 1 &&
           a->num_heads >= 1 && a->total_tokens >= 0;
}

// The fused schedule runs each (sequence, head) serially in one workgroup, one
// workgroup per compute unit at a time, so its time follows the larger of the
// longest sequence and the mean load per compute unit (in 16-token sub-chunks).
// When the longest sequence is more than 1.8 times that mean (the crossover
// measured on ragged batches of 384 to 1024 pairs), the two-pass schedule, whose
// only serial part is the state recurrence, is the faster one.  Without the host
// copy of cu_seqlens the lengths are unknown here and the pair count decides.
constexpr int64_t kFusedCUs = 256;  // compute units of gfx950 (MI355X)
bool lengths_balanced(const kda_prefill_args *a) {
    if (!a->cu_seqlens_host) return true;
    int64_t jmax = 0, jsum = 0;
    for (int32_t n = 0; n < a->num_seqs; ++n) {
        const int64_t L = (int64_t)a->cu_seqlens_host[n + 1] - a->cu_seqlens_host[n];
        const int64_t J = L > 0 ? (L + 15) / 16 : 0;
        jmax = J > jmax ? J : jmax;
        jsum += J;
    }
    return 10 * jmax * kFusedCUs <= 18 * jsum * (int64_t)a->num_heads;
}

// The schedule a call runs: explicit, or chosen (the fused one for many pairs of
// balanced lengths, else two passes when a workspace is given, else one pass).
int resolve_schedule(const kda_prefill_args *a, bool with_workspace) {
    if (a->schedule != KDA_SCHEDULE_AUTO) return a->schedule;
    if (two_pass_applies(a) && (int64_t)a->num_seqs * a->num_heads >= KDA_FUSED_MIN_PAIRS && lengths_balanced(a))
        return KDA_SCHEDULE_FUSED;
    return two_pass_applies(a) && with_workspace ? KDA_SCHEDULE_TWO_PASS : KDA_SCHEDULE_ONE_PASS;
}

// Most 16-token sub-chunks of any sequence: from the host copy of cu_seqlens
// when given (already validated), else an upper bound.
int64_t max_subchunks(const kda_prefill_args *a) {
    if (a->cu_seqlens_host) {
        int64_t m = 0;
        for (int32_t n = 0; n < a->num_seqs; ++n) {
            const int64_t L = (int64_t)a->cu_seqlens_host[n + 1] - a->cu_seqlens_host[n];
            m = L > m ? L : m;
        }
        return (m + 15) / 16;
    }
    if (!a->cu_seqlens) return (a->total_tokens / a->num_seqs + 15) / 16;
    return (a->total_tokens + 15) / 16;
}

// Sub-chunks per sequence per window that `bytes` of workspace hold (0: none).
int64_t window_subchunks(const kda_prefill_args *a, size_t bytes) {
    const size_t carry = kda::split_carry_bytes(a->num_seqs, a->num_heads);
    const size_t per = kda::split_window_bytes(a->num_seqs, a->num_heads, 1) - carry;
    return bytes > carry ? (int64_t)((bytes - carry) / per) : 0;
}

}  // namespace

namespace kda {

// Launch log: one line per kernel launch on stderr when the environment variable
// KDA_TRACE is set to a nonzero value when the library first launches (grid,
// block, dynamic LDS and the instantiation; no numerics).
bool trace_on() {
    static const bool on = [] {
        const char *v = std::getenv("KDA_TRACE");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

void trace(const char *fmt, ...) {
    if (!trace_on()) return;
    char line[384];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(line, sizeof(line), fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "[kda] %s\n", line);
}

constexpr int kDefaultSpinLimit = 1 << 22;
std::atomic<int> g_spin_limit{kDefaultSpinLimit};
int spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

}  // namespace kda

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int32_t kda_set_spin_limit(int32_t polls) {
    return kda::g_spin_limit.exchange(polls > 0 ? polls : kda::kDefaultSpinLimit);
}

const char *kda_status_string(kda_status s) {
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
    const size_t csb = (size_t)num_seqs * 3 * channels * esize(dtype);
    if (conv_state_out && conv_state_out != conv_state_in &&
        overlap(conv_state_out, csb, conv_state_in, csb))
        return fail(KDA_ERR_INVALID_ARG, "conv_state_out partially overlaps conv_state_in");
    const Buf bufs[] = {{y, bytes, "y"}, {conv_state_out, conv_state_out ? csb : 0, "conv_state_out"},
                        {x, bytes, "x"}, {weight, (size_t)channels * 16, "weight"},
                        {bias, bias ? (size_t)channels * 4 : 0, "bias"},
                        {conv_state_in, conv_state_out == conv_state_in ? 0 : csb, "conv_state_in"},
                        {cu_seqlens, cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0, "cu_seqlens"}};
    st = check_written(bufs, 7, 2);
    if (st != KDA_OK) return st;
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
    if (!two_pass_applies(a) || resolve_schedule(a, true) != KDA_SCHEDULE_TWO_PASS) return 0;
    const size_t full = kda::split_workspace_bytes(a->total_tokens, a->num_seqs, a->num_heads);
    if (full <= KDA_PREFILL_WORKSPACE_CAP) return full;
    int64_t jw = window_subchunks(a, KDA_PREFILL_WORKSPACE_CAP);
    if (jw < 1) jw = 1;
    const int64_t mj = max_subchunks(a);
    if (jw > mj) jw = mj > 0 ? mj : 1;
    const size_t win = kda::split_window_bytes(a->num_seqs, a->num_heads, jw);
    return win < full ? win : full;
}

size_t kda_prefill_workspace_full_size(const kda_prefill_args *a) {
    if (!two_pass_applies(a)) return 0;
    return kda::split_workspace_bytes(a->total_tokens, a->num_seqs, a->num_heads);
}

size_t kda_prefill_workspace_min_size(const kda_prefill_args *a) {
    if (!two_pass_applies(a)) return 0;
    const size_t full = kda::split_workspace_bytes(a->total_tokens, a->num_seqs, a->num_heads);
    const size_t one = kda::split_window_bytes(a->num_seqs, a->num_heads, 1);
    return one < full ? one : full;
}

}  // extern "C"

namespace {

// kda_prefill's checks and launches, with the workspace the caller's or the
// scratch array's (kda_prefill_noalloc).
kda_status prefill_impl(const kda_prefill_args *a, hipStream_t stream) {
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
    size_t rows = 0;
    st = pool_rows(a->state_slots, a->num_slots, a->num_seqs, rows);
    if (st != KDA_OK) return st;
    const size_t sb = rows * H * 128 * 128 * state_esize(a->flags);
    const size_t csb = rows * 3 * 3 * H * 128 * es;
    if (a->state_out && (const void *)a->state_out != (const void *)a->state_in &&
        overlap(a->state_out, sb, a->state_in, sb))
        return fail(KDA_ERR_INVALID_ARG, "state_out partially overlaps state_in");
    if (a->conv_state_out && a->conv_state_out != a->conv_state_in &&
        overlap(a->conv_state_out, csb, a->conv_state_in, csb))
        return fail(KDA_ERR_INVALID_ARG, "conv_state_out partially overlaps conv_state_in");
    // schedule; windows when a two-pass workspace holds less than the whole call
    if (a->schedule < KDA_SCHEDULE_AUTO || a->schedule > KDA_SCHEDULE_FUSED)
        return fail(KDA_ERR_INVALID_ARG, "schedule %d: use a KDA_SCHEDULE_* value", a->schedule);
    const int sched = resolve_schedule(a, a->workspace != nullptr);
    if ((sched == KDA_SCHEDULE_TWO_PASS || sched == KDA_SCHEDULE_FUSED) && !two_pass_applies(a))
        return fail(KDA_ERR_UNSUPPORTED, "the %s schedule needs bf16 I/O and chunk_size 0 or 16",
                    sched == KDA_SCHEDULE_FUSED ? "fused" : "two-pass");
    if (sched == KDA_SCHEDULE_TWO_PASS && !a->workspace)
        return fail(KDA_ERR_INVALID_ARG, "the two-pass schedule needs a workspace "
                                         "(kda_prefill_workspace_size)");
    const bool two_pass = sched == KDA_SCHEDULE_TWO_PASS;
    const bool fused = sched == KDA_SCHEDULE_FUSED;
    kda::SplitPlan plan{0, 1};
    if (two_pass) {
        const size_t need_min = kda_prefill_workspace_min_size(a);
        if (a->workspace_bytes < need_min)
            return fail(KDA_ERR_INVALID_ARG, "workspace of %zu bytes: the two-pass schedule needs at least "
                                             "%zu (kda_prefill_workspace_min_size)", a->workspace_bytes, need_min);
        const size_t full = kda::split_workspace_bytes(T, a->num_seqs, a->num_heads);
        if (a->workspace_bytes < full) {
            const int64_t mj = max_subchunks(a);
            int64_t jw = window_subchunks(a, a->workspace_bytes);
            if (jw > mj) jw = mj;
            if (jw < 1) jw = 1;
            plan.jw = jw;
            plan.windows = mj > 0 ? (mj + jw - 1) / jw : 1;
        }
    }
    const size_t wb = two_pass ? a->workspace_bytes : 0;
    const int N = a->num_seqs;
    const size_t CC = (size_t)3 * H * 128;
    // Every written buffer (o, state_out, conv_state_out, workspace) against every
    // other buffer.  state_out may equal state_in and conv_state_out may equal
    // conv_state_in (in-place update); those two pairs were checked above.
    const bool sio = a->state_out && (const void *)a->state_out == (const void *)a->state_in;
    const bool cio = a->conv_state_out && a->conv_state_out == a->conv_state_in;
    const Buf bufs[] = {{a->o, tok, "o"}, {a->state_out, sb, "state_out"},
                        {a->conv_state_out, csb, "conv_state_out"},
                        {two_pass ? a->workspace : nullptr, wb, "workspace"},
                        {a->q, tok, "q"}, {a->k, tok, "k"}, {a->v, tok, "v"}, {a->gate, tok, "gate"},
                        {a->beta, (size_t)T * H * es, "beta"}, {a->conv_weight, CC * 16, "conv_weight"},
                        {a->conv_bias, a->conv_bias ? CC * 4 : 0, "conv_bias"},
                        {a->state_in, sio ? 0 : sb, "state_in"},
                        {a->conv_state_in, cio ? 0 : csb, "conv_state_in"},
                        {a->cu_seqlens, a->cu_seqlens ? (size_t)(N + 1) * 4 : 0, "cu_seqlens"},
                        {a->state_slots, a->state_slots ? (size_t)N * 4 : 0, "state_slots"}};
    st = check_written(bufs, 15, 4);
    if (st != KDA_OK) return st;

    kda_prefill_args args = *a;
    if (args.scale == 0.f) args.scale = 1.0f / std::sqrt(128.0f);
    const int64_t pairs = (int64_t)a->num_seqs * H;
    // dv tile per workgroup: enough workgroups for 256 compute units.  The tile
    // changes only which workgroup computes a column, not the arithmetic.
    int dv_tile = pairs >= 256 ? 128 : (pairs >= 128 ? 64 : 32);
    // The two-pass schedule's wide pass B (all 128 columns per workgroup) serves
    // throughput; when one sequence dominates (lengths_balanced), the recurrence of
    // that sequence sets the time, and the narrow pass B (two 16-column tiles per
    // workgroup, a shorter step) is faster: 1 x 65,536 + 5 x 256 tokens at 64
    // heads ran 3.48 ms narrow against 5.67 ms wide.
    if (two_pass && dv_tile == 128 && !lengths_balanced(a)) dv_tile = 32;
    if (fused && a->dv_tile != 0 && a->dv_tile != 128)
        return fail(KDA_ERR_UNSUPPORTED, "dv_tile %d: the fused schedule takes 0 or 128", a->dv_tile);
    if (a->dv_tile != 0) {
        if (!(a->dv_tile == 32 || a->dv_tile == 64 || a->dv_tile == 128 ||
              (two_pass && a->dv_tile == 16)))
            return fail(KDA_ERR_UNSUPPORTED, "dv_tile %d: use 0, 32, 64 or 128 (16 with the "
                                             "two-pass schedule)", a->dv_tile);
        dv_tile = a->dv_tile;
    }
    hipError_t e;
    if (fused) {
        e = kda::launch_prefill_fused(&args, stream);
    } else if (two_pass) {
        e = kda::launch_prefill_split(&args, dv_tile, plan, stream);
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


// Scratch of kda_prefill_noalloc: one array per GPU the library runs on, held
// until the process ends.  Host code uses only the address that
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[KDA_PREFILL_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

kda_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill(const kda_prefill_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    return prefill_impl(a, stream);
}

kda_status kda_prefill_noalloc(const kda_prefill_args *a, hipStream_t stream) {
    g_err[0] = 0;
    if (!a) return fail(KDA_ERR_INVALID_ARG, "args is NULL");
    if (a->workspace || a->workspace_bytes)
        return fail(KDA_ERR_INVALID_ARG, "kda_prefill_noalloc takes no workspace (workspace must be NULL, "
                                         "workspace_bytes 0)");
    kda_prefill_args args = *a;
    if (two_pass_applies(a) && resolve_schedule(a, true) == KDA_SCHEDULE_TWO_PASS) {
        const size_t need = kda_prefill_workspace_min_size(a);
        if (need > KDA_PREFILL_SCRATCH_BYTES)
            return fail(KDA_ERR_INVALID_ARG, "this call needs at least %zu bytes of two-pass workspace; the "
                                             "scratch of kda_prefill_noalloc holds %zu (use kda_prefill with a "
                                             "workspace)", need, (size_t)KDA_PREFILL_SCRATCH_BYTES);
        kda_status st = check_common(a->num_seqs, a->num_heads, a->head_dim_k, a->head_dim_v, a->dtype,
                                     a->flags, a->scale, a->gate_lower_bound);
        if (st != KDA_OK) return st;
        st = scratch_address(&args.workspace);
        if (st != KDA_OK) return st;
        args.workspace_bytes = KDA_PREFILL_SCRATCH_BYTES;
    }
    return prefill_impl(&args, stream);
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
    const size_t CC = (size_t)3 * a->num_heads * 128;
    const Buf bufs[] = {{a->o, tok, "o"}, {a->state, sb, "state"}, {a->conv_state, cb, "conv_state"},
                        {a->q, tok, "q"}, {a->k, tok, "k"}, {a->v, tok, "v"}, {a->gate, tok, "gate"},
                        {a->beta, tok / 128, "beta"}, {a->conv_weight, CC * 16, "conv_weight"},
                        {a->conv_bias, a->conv_bias ? CC * 4 : 0, "conv_bias"},
                        {a->state_slots, a->state_slots ? (size_t)a->num_seqs * 4 : 0, "state_slots"}};
    st = check_written(bufs, 11, 3);
    if (st != KDA_OK) return st;
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
    const size_t CC = (size_t)3 * a->num_heads * 128;
    // state and conv_state are written only by a pending commit, but are always
    // treated as written
    const Buf bufs[] = {{a->o, tok, "o"}, {a->updates, rb, "updates"}, {a->state, sb, "state"},
                        {a->conv_state, cb, "conv_state"},
                        {a->q, tok, "q"}, {a->k, tok, "k"}, {a->v, tok, "v"}, {a->gate, tok, "gate"},
                        {a->beta, tok / 128, "beta"}, {a->conv_weight, CC * 16, "conv_weight"},
                        {a->conv_bias, a->conv_bias ? CC * 4 : 0, "conv_bias"},
                        {a->pending_updates, pb, "pending_updates"},
                        {a->pending_accepted, a->pending_updates ? (size_t)a->num_seqs * 4 : 0,
                         "pending_accepted"},
                        {a->state_slots, a->state_slots ? (size_t)a->num_seqs * 4 : 0, "state_slots"}};
    st = check_written(bufs, 14, 4);
    if (st != KDA_OK) return st;
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
    const Buf bufs[] = {{a->state, sb, "state"}, {a->conv_state, cb, "conv_state"},
                        {a->updates, rb, "updates"}, {a->accepted, (size_t)a->num_seqs * 4, "accepted"},
                        {a->state_slots, a->state_slots ? (size_t)a->num_seqs * 4 : 0, "state_slots"}};
    st = check_written(bufs, 5, 2);
    if (st != KDA_OK) return st;
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
    // the slot lists must survive the writes into the destination pools
    const size_t lb = (size_t)a->count * 4;
    const Buf bufs[] = {{a->state_dst, sb, "state_dst"}, {a->conv_dst, a->conv_dst ? cb : 0, "conv_dst"},
                        {a->src_slots, lb, "src_slots"}, {a->dst_slots, lb, "dst_slots"}};
    st = check_written(bufs, 4, 2);
    if (st != KDA_OK) return st;
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
