// kda_internal.h -- host-side launch entry points of the individual kernels.
// Arguments are validated by the C ABI layer (kda_api.hip) before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Launch log (KDA_TRACE=1 in the environment): one stderr line per launch with
// the kernel, its grid, block and dynamic LDS.
bool trace_on();
void trace(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

// Polls of a fused-prefill hand-over wait before it gives up (kda_set_spin_limit).
int spin_limit();

// Conv over packed sequences; x, y: [T][channels].
hipError_t launch_short_conv(kda_dtype dt, const void *x, void *y, int64_t T, int channels,
                             const float *w, const float *b, const void *cs_in,
                             const int32_t *cu, int num_seqs, bool silu, hipStream_t s);

// Last three raw tokens of (conv_state_in ++ sequence) for up to three sources that
// together form the conv channels: source i has `ch[i]` channels and rows of `ch[i]`
// elements ([T][ch[i]]).  Writes cs_out [rows][3][sum ch]; cs_out may alias cs_in.
// Sequence n uses row slots[n] (skipped when outside [0, num_slots)), or row n
// when slots is null.
hipError_t launch_conv_tail(kda_dtype dt, const void *const src[3], const int ch[3],
                            int64_t T, const void *cs_in, void *cs_out, const int32_t *cu,
                            int num_seqs, const int32_t *slots, int num_slots, hipStream_t s);

// Gate and beta in-projections (two matrix-core passes through the workspace).
size_t gate_proj_workspace_bytes(int64_t T, int H);
hipError_t launch_gate_proj(const kda_gate_beta_args *a, hipStream_t s);

// Pool rows: state (and conv state when given) of slot src[i] -> slot dst[i].
hipError_t launch_state_copy(const kda_state_copy_args *a, hipStream_t s);

struct PrefillLaunch {
    const kda_prefill_args *a;
    int chunk;      // 16, 32 or 64
    int dv_tile;    // dv columns per workgroup: 32, 64 or 128
};
hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t s);

hipError_t launch_decode(const kda_decode_args *a, hipStream_t s);
hipError_t launch_decode_multi(const kda_decode_multi_args *a, hipStream_t s);
hipError_t launch_decode_commit(const kda_decode_commit_args *a, hipStream_t s);

// Two-pass prefill (bf16 I/O, 16-token sub-chunks).  Workspace for the whole call
// in one window (packed slots), and for windows of jw sub-chunks per sequence
// (the window's records, then the fp32 carry of every (sequence, head) state).
size_t split_workspace_bytes(int64_t total_tokens, int num_seqs, int H);
size_t split_window_bytes(int num_seqs, int H, int64_t jw);
size_t split_carry_bytes(int num_seqs, int H);
struct SplitPlan {
    int64_t jw;       // sub-chunks per sequence per window; 0: one window, packed slots
    int64_t windows;  // windows to run when jw > 0
};
hipError_t launch_prefill_split(const kda_prefill_args *a, int dv_tile, const SplitPlan &plan, hipStream_t s);
// Fused schedule: one workgroup per (sequence, head), no workspace.
hipError_t launch_prefill_fused(const kda_prefill_args *a, hipStream_t s);

}  // namespace kda
