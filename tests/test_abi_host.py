"""Host-side tests of the C ABI (no GPU): the library loads, exports every symbol
include/kda.h declares, and rejects bad arguments on the host before touching a
device.  The validation paths return before any HIP call, so they run here."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_short_amd as pkg
from gated_delta_rule_short_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from gated_delta_rule_short_amd import _build
        _build.build()
    return K.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text))


def test_header_and_binding_agree():
    assert _declared_functions() == set(K.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.kda_abi_version() == 4


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(1) == b"KDA_ERR_INVALID_ARG"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(3) == b"KDA_ERR_HIP"


def test_struct_layouts_match_header():
    # offsets of the first pointer fields follow the C layout rules (int64 aligned at 8)
    assert K.KdaPrefillArgs.total_tokens.offset == 24
    assert K.KdaPrefillArgs.q.offset == 48
    assert K.KdaPrefillArgs.state_slots.offset == 48 + 16 * 8
    assert ctypes.sizeof(K.KdaPrefillArgs) == 48 + 18 * 8
    assert K.KdaDecodeArgs.q.offset == 32
    assert K.KdaDecodeArgs.state_slots.offset == 32 + 10 * 8
    assert ctypes.sizeof(K.KdaDecodeArgs) == 32 + 12 * 8
    assert K.KdaDecodeMultiArgs.q.offset == 40
    assert K.KdaDecodeMultiArgs.pending_tokens.offset == 40 + 13 * 8
    assert K.KdaDecodeMultiArgs.state_slots.offset == 40 + 14 * 8
    assert ctypes.sizeof(K.KdaDecodeMultiArgs) == 40 + 16 * 8
    assert K.KdaDecodeCommitArgs.accepted.offset == 32
    assert ctypes.sizeof(K.KdaDecodeCommitArgs) == 32 + 6 * 8
    assert K.KdaStateCopyArgs.src_slots.offset == 32
    assert ctypes.sizeof(K.KdaStateCopyArgs) == 32 + 6 * 8


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def _prefill_args(**kw):
    a = K.KdaPrefillArgs(num_seqs=1, num_heads=2, head_dim_k=128, head_dim_v=128, chunk_size=0,
                         total_tokens=64, dtype=K.KDA_BF16, flags=0, scale=0.0,
                         gate_lower_bound=-5.0)
    for f in ("q", "k", "v", "gate", "beta", "conv_weight", "o"):
        setattr(a, f, None)
    base = 0x100000
    for i, f in enumerate(("q", "k", "v", "gate", "beta", "conv_weight", "o")):
        setattr(a, f, ctypes.c_void_p(base + i * 0x1000000))
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("num_seqs", 0, K.KDA_ERR_INVALID_ARG),
    ("num_heads", 0, K.KDA_ERR_INVALID_ARG),
    ("head_dim_k", 64, K.KDA_ERR_UNSUPPORTED),
    ("head_dim_v", 256, K.KDA_ERR_UNSUPPORTED),
    ("chunk_size", 48, K.KDA_ERR_UNSUPPORTED),
    ("flags", 16, K.KDA_ERR_UNSUPPORTED),
    ("dtype", 7, K.KDA_ERR_INVALID_ARG),
    ("gate_lower_bound", 0.0, K.KDA_ERR_INVALID_ARG),
    ("gate_lower_bound", float("nan"), K.KDA_ERR_INVALID_ARG),
    ("scale", -1.0, K.KDA_ERR_INVALID_ARG),
    ("total_tokens", -1, K.KDA_ERR_INVALID_ARG),
    ("total_tokens", 1 << 31, K.KDA_ERR_INVALID_ARG),
    ("q", None, K.KDA_ERR_INVALID_ARG),
    ("conv_weight", None, K.KDA_ERR_INVALID_ARG),
])
def test_prefill_rejects_bad_arguments(lib, field, value, status):
    a = _prefill_args(**{field: value})
    assert lib.kda_prefill(ctypes.byref(a), None) == status
    assert lib.kda_last_error() != b""


def test_prefill_fp32_chunk64_unsupported(lib):
    a = _prefill_args(dtype=K.KDA_F32, chunk_size=64)
    assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_UNSUPPORTED


def test_prefill_checks_host_cu_seqlens(lib):
    for cu in ([1, 64], [0, 30, 20, 64], [0, 63]):
        arr = (ctypes.c_int32 * len(cu))(*cu)
        a = _prefill_args(num_seqs=len(cu) - 1, cu_seqlens=FAKE,
                          cu_seqlens_host=ctypes.cast(arr, ctypes.c_void_p))
        assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG, cu


def test_prefill_dense_layout_needs_divisible_tokens(lib):
    a = _prefill_args(num_seqs=3, total_tokens=64)
    assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_prefill_rejects_output_overlapping_input(lib):
    a = _prefill_args()
    a.o = a.q
    assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_prefill_rejects_partial_state_alias(lib):
    a = _prefill_args(state_in=ctypes.c_void_p(0x9000000), state_out=ctypes.c_void_p(0x9000010))
    assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def _decode_args(**kw):
    a = K.KdaDecodeArgs(num_seqs=2, num_heads=2, head_dim_k=128, head_dim_v=128,
                        dtype=K.KDA_BF16, flags=0, scale=0.0, gate_lower_bound=-5.0)
    base = 0x100000
    for i, f in enumerate(("q", "k", "v", "gate", "beta", "conv_weight", "conv_state", "state",
                           "o")):
        setattr(a, f, ctypes.c_void_p(base + i * 0x1000000))
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("num_seqs", -1, K.KDA_ERR_INVALID_ARG),
    ("head_dim_k", 32, K.KDA_ERR_UNSUPPORTED),
    ("flags", 0x10, K.KDA_ERR_UNSUPPORTED),
    ("state", None, K.KDA_ERR_INVALID_ARG),
    ("conv_state", None, K.KDA_ERR_INVALID_ARG),
    ("o", None, K.KDA_ERR_INVALID_ARG),
    ("gate_lower_bound", 1.0, K.KDA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(lib, field, value, status):
    a = _decode_args(**{field: value})
    assert lib.kda_decode(ctypes.byref(a), None) == status


def test_decode_state_overlap_size_follows_storage(lib):
    # every case here is rejected before a launch (the pointers are fake)
    bf16_bytes = 2 * 2 * 128 * 128 * 2
    a = _decode_args(flags=K.KDA_F_STATE_BF16)
    a.o = ctypes.c_void_p(a.state + bf16_bytes - 2)  # last element of a bf16 state
    assert lib.kda_decode(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _decode_args()
    a.o = ctypes.c_void_p(a.state + bf16_bytes)  # inside an fp32 state of the same shape
    assert lib.kda_decode(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_decode_rejects_state_overlapping_output(lib):
    a = _decode_args()
    a.state = a.o
    assert lib.kda_decode(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def _multi_args(**kw):
    a = K.KdaDecodeMultiArgs(num_seqs=2, num_heads=2, head_dim_k=128, head_dim_v=128,
                             num_tokens=6, dtype=K.KDA_BF16, flags=0, scale=0.0,
                             gate_lower_bound=-5.0)
    base = 0x100000
    for i, f in enumerate(("q", "k", "v", "gate", "beta", "conv_weight", "conv_state", "state",
                           "o", "updates")):
        setattr(a, f, ctypes.c_void_p(base + i * 0x1000000))
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("num_tokens", 0, K.KDA_ERR_INVALID_ARG),
    ("num_tokens", K.MAX_SPEC_TOKENS + 1, K.KDA_ERR_INVALID_ARG),
    ("head_dim_v", 64, K.KDA_ERR_UNSUPPORTED),
    ("updates", None, K.KDA_ERR_INVALID_ARG),
    ("state", None, K.KDA_ERR_INVALID_ARG),
    ("flags", 0x40, K.KDA_ERR_UNSUPPORTED),
    ("pending_updates", ctypes.c_void_p(0x70000000), K.KDA_ERR_INVALID_ARG),  # no counts
])
def test_decode_multi_rejects_bad_arguments(lib, field, value, status):
    a = _multi_args(**{field: value})
    assert lib.kda_decode_multi(ctypes.byref(a), None) == status
    assert lib.kda_last_error() != b""


def test_decode_multi_rejects_overlaps(lib):
    a = _multi_args()
    a.updates = a.state  # records over the state
    assert lib.kda_decode_multi(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _multi_args(pending_accepted=ctypes.c_void_p(0x71000000), pending_tokens=6)
    a.pending_updates = ctypes.c_void_p(a.updates + 64)  # overlaps this call's records
    assert lib.kda_decode_multi(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _multi_args(pending_updates=ctypes.c_void_p(0x70000000),
                    pending_accepted=ctypes.c_void_p(0x71000000), pending_tokens=9)
    assert lib.kda_decode_multi(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def _commit_args(**kw):
    a = K.KdaDecodeCommitArgs(num_seqs=2, num_heads=2, head_dim_k=128, head_dim_v=128,
                              num_tokens=6, dtype=K.KDA_BF16)
    for i, f in enumerate(("accepted", "updates", "conv_state", "state")):
        setattr(a, f, ctypes.c_void_p(0x100000 + i * 0x1000000))
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("num_seqs", 0, K.KDA_ERR_INVALID_ARG),
    ("num_tokens", 9, K.KDA_ERR_INVALID_ARG),
    ("head_dim_k", 256, K.KDA_ERR_UNSUPPORTED),
    ("accepted", None, K.KDA_ERR_INVALID_ARG),
    ("updates", None, K.KDA_ERR_INVALID_ARG),
    ("dtype", 5, K.KDA_ERR_INVALID_ARG),
    ("flags", K.KDA_F_SILU, K.KDA_ERR_UNSUPPORTED),
])
def test_decode_commit_rejects_bad_arguments(lib, field, value, status):
    a = _commit_args(**{field: value})
    assert lib.kda_decode_commit(ctypes.byref(a), None) == status


def test_decode_commit_rejects_records_over_state(lib):
    a = _commit_args()
    a.updates = ctypes.c_void_p(a.state + 4096)
    assert lib.kda_decode_commit(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_pool_needs_num_slots(lib):
    # a slot map without a pool size is rejected on the host (no launch)
    a = _prefill_args(state_slots=FAKE, num_slots=0)
    assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _decode_args(state_slots=FAKE, num_slots=0)
    assert lib.kda_decode(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _multi_args(state_slots=FAKE, num_slots=-3)
    assert lib.kda_decode_multi(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _commit_args(state_slots=FAKE, num_slots=0)
    assert lib.kda_decode_commit(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_pool_size_drives_overlap_checks(lib):
    # with 9 pool rows the fp32 state of 2 heads spans 9 * 2 * 64 KiB: o inside it is rejected
    a = _decode_args(state_slots=FAKE, num_slots=9)
    a.o = ctypes.c_void_p(a.state + 8 * 2 * 65536)
    assert lib.kda_decode(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def _copy_args(**kw):
    a = K.KdaStateCopyArgs(count=2, num_heads=2, head_dim_k=128, head_dim_v=128, num_slots=4,
                           dtype=K.KDA_BF16, flags=0)
    for i, f in enumerate(("src_slots", "dst_slots", "state_src", "state_dst", "conv_src",
                           "conv_dst")):
        setattr(a, f, ctypes.c_void_p(0x100000 + i * 0x1000000))
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("count", -1, K.KDA_ERR_INVALID_ARG),
    ("num_slots", 0, K.KDA_ERR_INVALID_ARG),
    ("num_heads", 0, K.KDA_ERR_INVALID_ARG),
    ("head_dim_k", 64, K.KDA_ERR_UNSUPPORTED),
    ("flags", K.KDA_F_SILU, K.KDA_ERR_UNSUPPORTED),
    ("src_slots", None, K.KDA_ERR_INVALID_ARG),
    ("state_dst", None, K.KDA_ERR_INVALID_ARG),
    ("conv_dst", None, K.KDA_ERR_INVALID_ARG),  # conv_src given without conv_dst
])
def test_state_copy_rejects_bad_arguments(lib, field, value, status):
    a = _copy_args(**{field: value})
    assert lib.kda_state_copy(ctypes.byref(a), None) == status


def test_state_copy_rejects_partial_pool_overlap(lib):
    a = _copy_args()
    a.state_dst = ctypes.c_void_p(a.state_src + 4096)
    assert lib.kda_state_copy(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_state_copy_of_nothing_is_ok(lib):
    a = _copy_args(count=0)  # validated, then nothing is launched
    assert lib.kda_state_copy(ctypes.byref(a), None) == K.KDA_OK


def _gb_args(**kw):
    a = K.KdaGateBetaArgs(total_tokens=64, hidden=256, rank=128, num_heads=64, head_dim_k=128,
                          flags=0, gate_lower_bound=-5.0)
    for i, f in enumerate(("x", "w_a", "w_b", "w_beta", "gate", "beta", "workspace")):
        setattr(a, f, ctypes.c_void_p(0x100000 + i * 0x1000000))
    a.workspace_bytes = 16 * 64 * (128 + 64) + 2 * 64 * 128
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("total_tokens", -1, K.KDA_ERR_INVALID_ARG),
    ("hidden", 200, K.KDA_ERR_UNSUPPORTED),
    ("hidden", 384, K.KDA_ERR_UNSUPPORTED),  # a multiple of 128 but not of 256
    ("rank", 64, K.KDA_ERR_UNSUPPORTED),
    ("num_heads", 48, K.KDA_ERR_UNSUPPORTED),
    ("num_heads", 96, K.KDA_ERR_UNSUPPORTED),
    ("head_dim_k", 64, K.KDA_ERR_UNSUPPORTED),
    ("flags", K.KDA_F_SILU, K.KDA_ERR_UNSUPPORTED),
    ("gate_lower_bound", 0.5, K.KDA_ERR_INVALID_ARG),
    ("x", None, K.KDA_ERR_INVALID_ARG),
    ("w_b", ctypes.c_void_p(0x2000008), K.KDA_ERR_INVALID_ARG),  # not 16-byte aligned
    ("workspace_bytes", 1024, K.KDA_ERR_INVALID_ARG),
])
def test_gate_beta_rejects_bad_arguments(lib, field, value, status):
    a = _gb_args(**{field: value})
    assert lib.kda_gate_beta_proj(ctypes.byref(a), None) == status


def test_gate_beta_rejects_overlaps_and_sizes_workspace(lib):
    a = _gb_args()
    a.gate = a.x  # output over an input
    assert lib.kda_gate_beta_proj(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    a = _gb_args()
    a.beta = ctypes.c_void_p(a.workspace + 16)
    assert lib.kda_gate_beta_proj(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    assert lib.kda_gate_beta_workspace_size(ctypes.byref(_gb_args())) == 16 * 64 * (128 + 64) + 2 * 64 * 128
    assert lib.kda_gate_beta_proj(ctypes.byref(_gb_args(total_tokens=0)), None) == K.KDA_OK


def test_short_conv_rejects_bad_arguments(lib):
    f = lib.kda_short_conv
    # num_seqs 0
    assert f(FAKE, ctypes.c_void_p(0x900000), 8, 4, FAKE, None, None, None, None, None, 0, 1, 0,
             None) == K.KDA_ERR_INVALID_ARG
    # unknown flag
    assert f(FAKE, ctypes.c_void_p(0x900000), 8, 4, FAKE, None, None, None, None, None, 1, 1, 2,
             None) == K.KDA_ERR_UNSUPPORTED
    # y overlapping x
    assert f(FAKE, FAKE, 8, 4, FAKE, None, None, None, None, None, 1, 1, 0,
             None) == K.KDA_ERR_INVALID_ARG
    # bad host cu_seqlens
    cu = (ctypes.c_int32 * 3)(0, 5, 7)
    assert f(FAKE, ctypes.c_void_p(0x900000), 8, 4, FAKE, None, None, None, FAKE,
             ctypes.cast(cu, ctypes.c_void_p), 2, 1, 0, None) == K.KDA_ERR_INVALID_ARG


def test_workspace_size_query(lib):
    a = _prefill_args(total_tokens=4096, num_heads=64)
    need = lib.kda_prefill_workspace_size(ctypes.byref(a))
    assert need == 64 * (4096 // 16 + 1) * 17408
    a.chunk_size = 64
    assert lib.kda_prefill_workspace_size(ctypes.byref(a)) == 0
    b = _prefill_args(dtype=K.KDA_F32)
    assert lib.kda_prefill_workspace_size(ctypes.byref(b)) == 0


def test_prefill_rejects_workspace_overlapping_output(lib):
    a = _prefill_args(total_tokens=64, num_heads=2)
    a.workspace = a.o
    a.workspace_bytes = lib.kda_prefill_workspace_size(ctypes.byref(a))
    assert lib.kda_prefill(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        K.load_library(str(tmp_path / "missing.so"))


def test_binding_checks_pool_rows_before_any_launch(lib):
    """The binding rejects pools of different sizes, a missing pool, and an allocated
    state_out with a slot map (the library would write past it); these fail before any
    device call, on CPU tensors."""
    import torch
    dev = torch.device("cpu")
    q = torch.zeros((4, 2, 128), dtype=torch.bfloat16)
    beta = torch.zeros((4, 2), dtype=torch.bfloat16)
    w = torch.zeros((3 * 2 * 128, 4))
    cu = torch.tensor([0, 4], dtype=torch.int32)
    slots = torch.zeros(1, dtype=torch.int32)
    pool = torch.zeros((5, 2, 128, 128))
    with pytest.raises(ValueError):
        K.kda_prefill(q, q, q, q, beta, w, cu_seqlens=cu, state_in=pool, state_out=True,
                      state_slots=slots)
    with pytest.raises(ValueError):
        K.kda_prefill(q, q, q, q, beta, w, cu_seqlens=cu, state_slots=slots)
    cpool = torch.zeros((3, 3, 3 * 2 * 128), dtype=torch.bfloat16)
    qd = torch.zeros((1, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        K.kda_decode(qd, qd, qd, qd, beta[:1], w, cpool, pool, state_slots=slots)
    with pytest.raises(ValueError):  # no slot map: one row per sequence
        K.kda_decode(qd, qd, qd, qd, beta[:1], w, cpool[:1], pool)
