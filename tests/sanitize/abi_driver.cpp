// Host-only sanitizer run of the C-ABI layer (test infrastructure): kda_api.hip's
// host code is compiled with AddressSanitizer and UndefinedBehaviorSanitizer
// against the stub launchers below, which record what would be launched instead
// of touching a GPU.  Every entry point is called with bad arguments (each must
// fail with its status and a message) and with good ones (each must reach its
// launcher), and the prefill's workspace planning is checked: the whole call at
// once when the workspace holds it, else windows of as many sub-chunks per
// sequence as fit beside the fp32 carry.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace kda {
static int g_launch = 0;
static SplitPlan g_plan{-1, -1};
static int g_dv = -1;
static const size_t kRecBytes = 13824, kCarry = 128 * 128 * 4;
hipError_t launch_short_conv(kda_dtype, const void *, void *, int64_t, int, const float *, const float *,
                             const void *, const int32_t *, int, bool, hipStream_t) { ++g_launch; return hipSuccess; }
hipError_t launch_conv_tail(kda_dtype, const void *const[3], const int[3], int64_t, const void *, void *,
                            const int32_t *, int, const int32_t *, int, hipStream_t) { ++g_launch; return hipSuccess; }
size_t gate_proj_workspace_bytes(int64_t T, int H) { return (size_t)4 * T * (128 + H) * 4 + (size_t)T * 128 * 2; }
hipError_t launch_gate_proj(const kda_gate_beta_args *, hipStream_t) { ++g_launch; return hipSuccess; }
hipError_t launch_state_copy(const kda_state_copy_args *, hipStream_t) { ++g_launch; return hipSuccess; }
hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t) { ++g_launch; g_dv = p.dv_tile; g_plan = {-2, -2}; return hipSuccess; }
hipError_t launch_decode(const kda_decode_args *, hipStream_t) { ++g_launch; return hipSuccess; }
hipError_t launch_decode_multi(const kda_decode_multi_args *, hipStream_t) { ++g_launch; return hipSuccess; }
hipError_t launch_decode_commit(const kda_decode_commit_args *, hipStream_t) { ++g_launch; return hipSuccess; }
size_t split_workspace_bytes(int64_t T, int N, int H) { return (size_t)H * (size_t)(T / 16 + N) * kRecBytes; }
size_t split_carry_bytes(int N, int H) { return (size_t)N * H * kCarry; }
size_t split_window_bytes(int N, int H, int64_t jw) { return (size_t)H * N * jw * kRecBytes + split_carry_bytes(N, H); }
hipError_t launch_prefill_split(const kda_prefill_args *, int dv, const SplitPlan &plan, hipStream_t) {
    ++g_launch; g_dv = dv; g_plan = plan; return hipSuccess;
}
hipError_t launch_prefill_fused(const kda_prefill_args *, hipStream_t) {
    ++g_launch; g_plan.jw = -3; return hipSuccess;
}
}  // namespace kda

static int failures = 0;
#define CHECK(cond, ...) do { if (!(cond)) { ++failures; std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
    std::fprintf(stderr, __VA_ARGS__); std::fprintf(stderr, " (%s)\n", kda_last_error()); } } while (0)

// fake device addresses, far apart: never dereferenced by the host code
static void *addr(int i) { return reinterpret_cast<void *>((uintptr_t)(i + 1) << 36); }

static kda_prefill_args prefill(int N, int H, int64_t T) {
    kda_prefill_args a;
    std::memset(&a, 0, sizeof(a));
    a.num_seqs = N; a.num_heads = H; a.head_dim_k = a.head_dim_v = 128; a.total_tokens = T;
    a.dtype = KDA_BF16; a.gate_lower_bound = -5.f;
    a.q = addr(0); a.k = addr(1); a.v = addr(2); a.gate = addr(3); a.beta = addr(4);
    a.conv_weight = (const float *)addr(5); a.o = addr(6);
    return a;
}

int main() {
    // ---- prefill: bad arguments
    {
        kda_prefill_args a = prefill(1, 2, 64);
        a.head_dim_k = 64; CHECK(kda_prefill(&a, nullptr) == KDA_ERR_UNSUPPORTED, "head dim");
        a = prefill(1, 2, 64); a.chunk_size = 48; CHECK(kda_prefill(&a, nullptr) == KDA_ERR_UNSUPPORTED, "chunk");
        a = prefill(1, 2, 64); a.o = const_cast<void *>(a.q); CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "o aliases q");
        a = prefill(1, 2, 64); a.dv_tile = 48; CHECK(kda_prefill(&a, nullptr) == KDA_ERR_UNSUPPORTED, "dv_tile");
        a = prefill(3, 2, 64); CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "dense layout 64 %% 3");
        int32_t bad_cu[3] = {0, 40, 20};
        a = prefill(2, 2, 64); a.cu_seqlens = (const int32_t *)addr(9); a.cu_seqlens_host = bad_cu;
        CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "host cu");
        a = prefill(1, 2, 64); a.workspace = addr(10); a.workspace_bytes = 1;
        CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "workspace below the minimum");
        a = prefill(1, 2, 64); a.state_in = addr(11); a.state_out = (char *)addr(11) + 16;
        CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "partial state alias");
        CHECK(kda_prefill(nullptr, nullptr) == KDA_ERR_INVALID_ARG, "null args");
        CHECK(kda_prefill_noalloc(nullptr, nullptr) == KDA_ERR_INVALID_ARG, "null args (noalloc)");
    }
    // ---- prefill: schedules and windows
    {
        const int N = 16, H = 64;
        std::vector<int32_t> cu(N + 1, 0);
        for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + 512 + 997 * n;  // the longest: 15,467 tokens
        const int64_t T = cu[N];
        kda_prefill_args a = prefill(N, H, T);
        a.cu_seqlens = (const int32_t *)addr(12);
        a.cu_seqlens_host = cu.data();
        a.state_in = addr(13); a.state_out = addr(14);
        kda::g_launch = 0;
        CHECK(kda_prefill(&a, nullptr) == KDA_OK && kda::g_plan.jw == -3, "1024 pairs: fused");
        CHECK(kda_prefill_workspace_size(&a) == 0, "the fused schedule needs no workspace");
        a.schedule = KDA_SCHEDULE_ONE_PASS;
        CHECK(kda_prefill(&a, nullptr) == KDA_OK && kda::g_plan.jw == -2, "explicit one pass");
        a.schedule = KDA_SCHEDULE_TWO_PASS;
        CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "two passes without a workspace");
        const size_t full = kda_prefill_workspace_full_size(&a);
        CHECK(full == (size_t)H * (T / 16 + N) * kda::kRecBytes, "full size");
        a.workspace = addr(15); a.workspace_bytes = full;
        CHECK(kda_prefill(&a, nullptr) == KDA_OK && kda::g_plan.jw == 0, "whole call in one window");
        CHECK(kda::g_dv == 128, "1024 pairs: 128 columns per workgroup (dv %d)", kda::g_dv);
        const size_t rec = kda_prefill_workspace_size(&a);
        CHECK(rec <= KDA_PREFILL_WORKSPACE_CAP && rec < full, "recommended size within the cap");
        a.workspace_bytes = rec;
        CHECK(kda_prefill(&a, nullptr) == KDA_OK, "recommended size runs");
        const int64_t maxj = (cu[N] - cu[N - 1] + 15) / 16;
        const int64_t jw = (int64_t)((rec - (size_t)N * H * 65536) / ((size_t)N * H * kda::kRecBytes));
        CHECK(kda::g_plan.jw == jw && kda::g_plan.windows == (maxj + jw - 1) / jw,
              "windows %lld x %lld (want %lld x %lld)", (long long)kda::g_plan.jw,
              (long long)kda::g_plan.windows, (long long)jw, (long long)((maxj + jw - 1) / jw));
        a.workspace_bytes = kda_prefill_workspace_min_size(&a);
        CHECK(kda_prefill(&a, nullptr) == KDA_OK && kda::g_plan.jw == 1 && kda::g_plan.windows == maxj,
              "minimum workspace: one sub-chunk per window");
        a.cu_seqlens_host = nullptr;  // without the host copy: plan for one sequence of all tokens
        CHECK(kda_prefill(&a, nullptr) == KDA_OK && kda::g_plan.windows == (T + 15) / 16, "upper bound");
        a.workspace = a.o;
        CHECK(kda_prefill(&a, nullptr) == KDA_ERR_INVALID_ARG, "workspace aliases o");
        a.workspace = nullptr; a.workspace_bytes = 0;
        kda_prefill_args b = a;
        b.workspace = addr(16); b.workspace_bytes = 64;
        CHECK(kda_prefill_noalloc(&b, nullptr) == KDA_ERR_INVALID_ARG, "noalloc takes no workspace");
    }
    // ---- decode family, conv, pool, projections
    {
        kda_decode_args d;
        std::memset(&d, 0, sizeof(d));
        d.num_seqs = 4; d.num_heads = 2; d.head_dim_k = d.head_dim_v = 128; d.dtype = KDA_BF16;
        d.gate_lower_bound = -5.f;
        d.q = addr(0); d.k = addr(1); d.v = addr(2); d.gate = addr(3); d.beta = addr(4);
        d.conv_weight = (const float *)addr(5); d.conv_state = addr(6); d.state = addr(7); d.o = addr(8);
        kda::g_launch = 0;
        CHECK(kda_decode(&d, nullptr) == KDA_OK && kda::g_launch == 1, "decode launches");
        d.o = d.state; CHECK(kda_decode(&d, nullptr) == KDA_ERR_INVALID_ARG, "o aliases state");
        d.o = addr(8); d.flags = 64; CHECK(kda_decode(&d, nullptr) == KDA_ERR_UNSUPPORTED, "flags");
        kda_decode_multi_args m;
        std::memset(&m, 0, sizeof(m));
        m.num_seqs = 4; m.num_heads = 2; m.head_dim_k = m.head_dim_v = 128; m.num_tokens = 6;
        m.dtype = KDA_BF16; m.gate_lower_bound = -5.f;
        m.q = addr(0); m.k = addr(1); m.v = addr(2); m.gate = addr(3); m.beta = addr(4);
        m.conv_weight = (const float *)addr(5); m.conv_state = addr(6); m.state = addr(7); m.o = addr(8);
        m.updates = (float *)addr(9);
        CHECK(kda_decode_multi(&m, nullptr) == KDA_OK, "multi launches");
        m.num_tokens = 9; CHECK(kda_decode_multi(&m, nullptr) == KDA_ERR_INVALID_ARG, "too many tokens");
        m.num_tokens = 6; m.pending_updates = m.updates; m.pending_accepted = (const int32_t *)addr(10);
        m.pending_tokens = 6; CHECK(kda_decode_multi(&m, nullptr) == KDA_ERR_INVALID_ARG, "pending aliases");
        kda_decode_commit_args c;
        std::memset(&c, 0, sizeof(c));
        c.num_seqs = 4; c.num_heads = 2; c.head_dim_k = c.head_dim_v = 128; c.num_tokens = 6; c.dtype = KDA_BF16;
        c.accepted = (const int32_t *)addr(0); c.updates = (const float *)addr(1);
        c.conv_state = addr(2); c.state = addr(3);
        CHECK(kda_decode_commit(&c, nullptr) == KDA_OK, "commit launches");
        c.state = (void *)c.updates; CHECK(kda_decode_commit(&c, nullptr) == KDA_ERR_INVALID_ARG, "alias");
        CHECK(kda_short_conv(addr(0), addr(1), 64, 384, (const float *)addr(2), nullptr, nullptr, nullptr,
                             nullptr, nullptr, 1, KDA_BF16, 0, nullptr) == KDA_OK, "conv launches");
        CHECK(kda_short_conv(addr(0), addr(0), 64, 384, (const float *)addr(2), nullptr, nullptr, nullptr,
                             nullptr, nullptr, 1, KDA_BF16, 0, nullptr) == KDA_ERR_INVALID_ARG, "conv alias");
        kda_state_copy_args s;
        std::memset(&s, 0, sizeof(s));
        s.count = 3; s.num_heads = 2; s.head_dim_k = s.head_dim_v = 128; s.num_slots = 8; s.dtype = KDA_BF16;
        s.src_slots = (const int32_t *)addr(0); s.dst_slots = (const int32_t *)addr(1);
        s.state_src = s.state_dst = addr(2);
        CHECK(kda_state_copy(&s, nullptr) == KDA_OK, "copy launches");
        s.dst_slots = (const int32_t *)addr(2); CHECK(kda_state_copy(&s, nullptr) == KDA_ERR_INVALID_ARG, "slots in pool");
        kda_gate_beta_args g;
        std::memset(&g, 0, sizeof(g));
        g.total_tokens = 64; g.hidden = 512; g.rank = 128; g.num_heads = 64; g.head_dim_k = 128;
        g.gate_lower_bound = -5.f;
        g.x = addr(0); g.w_a = addr(1); g.w_b = addr(2); g.w_beta = addr(3); g.gate = addr(4); g.beta = addr(5);
        g.workspace = addr(6); g.workspace_bytes = kda_gate_beta_workspace_size(&g);
        CHECK(kda_gate_beta_proj(&g, nullptr) == KDA_OK, "projection launches");
        g.hidden = 300; CHECK(kda_gate_beta_proj(&g, nullptr) == KDA_ERR_UNSUPPORTED, "hidden");
    }
    CHECK(std::strcmp(kda_status_string(KDA_ERR_HIP), "KDA_ERR_HIP") == 0, "status string");
    CHECK(std::strcmp(kda_status_string((kda_status)77), "KDA_UNKNOWN_STATUS") == 0, "unknown status");
    if (failures) return 1;
    std::printf("C-ABI sanitizer run ok\n");
    return 0;
}
