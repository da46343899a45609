"""MI355X (gfx950) implementation of the Kimi Delta Attention (KDA) sequence mixer.

The computation runs in libkda.so (hand-written HIP kernels behind the C ABI of
include/kda.h); this package is its thin Python binding.
"""
from .kda import (KDA_F32, KDA_BF16, KDA_F_SILU, KDA_F_NO_QK_L2NORM, KDA_F_GATE_IS_LOG,
                  KDA_F_STATE_BF16, PREFILL_WORKSPACE_CAP, PREFILL_SCRATCH_BYTES, SCHEDULES,
                  FUSED_MIN_PAIRS,
                  KdaError, MAX_SPEC_TOKENS, UPDATE_FLOATS, abi_version, kda_decode, kda_decode_commit,
                  kda_decode_multi, kda_gate_beta_proj, kda_prefill, kda_prefill_noalloc, kda_short_conv,
                  kda_state_copy, gate_beta_workspace_bytes, load_library,
                  prefill_workspace_bytes, load_calib_library, calib_state_rmw, calib_copy,
                  calib_fill, set_spin_limit)

__all__ = ["kda_short_conv", "kda_prefill", "kda_prefill_noalloc", "kda_decode", "kda_decode_multi",
           "kda_decode_commit", "kda_state_copy", "kda_gate_beta_proj",
           "gate_beta_workspace_bytes", "abi_version", "load_library",
           "prefill_workspace_bytes", "load_calib_library", "calib_state_rmw", "calib_copy",
           "calib_fill", "set_spin_limit",
           "KdaError", "MAX_SPEC_TOKENS", "UPDATE_FLOATS", "KDA_F32", "KDA_BF16", "KDA_F_SILU", "KDA_F_NO_QK_L2NORM",
           "KDA_F_GATE_IS_LOG", "KDA_F_STATE_BF16", "PREFILL_WORKSPACE_CAP",
           "PREFILL_SCRATCH_BYTES", "SCHEDULES", "FUSED_MIN_PAIRS"]
