"""ctypes binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream; every step of the mixer runs in the library's kernels.  There is no
fallback: if libkda.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1
KDA_F_SILU, KDA_F_NO_QK_L2NORM, KDA_F_GATE_IS_LOG, KDA_F_STATE_BF16 = 1, 2, 4, 8
PREFILL_WORKSPACE_CAP = 4 << 30  # KDA_PREFILL_WORKSPACE_CAP
PREFILL_SCRATCH_BYTES = 256 << 20  # KDA_PREFILL_SCRATCH_BYTES (kda_prefill_noalloc)

# every symbol include/kda.h declares
EXPORTS = ("kda_abi_version", "kda_set_spin_limit", "kda_status_string", "kda_last_error", "kda_short_conv",
           "kda_prefill", "kda_prefill_workspace_size", "kda_prefill_workspace_full_size",
           "kda_prefill_workspace_min_size", "kda_prefill_noalloc", "kda_decode", "kda_decode_multi",
           "kda_decode_commit", "kda_state_copy", "kda_gate_beta_proj",
           "kda_gate_beta_workspace_size")
MAX_SPEC_TOKENS = 8
UPDATE_FLOATS = 6 * 128  # floats per (sequence, head, token) update record

_c_i32, _c_i64, _c_u32, _c_f32, _p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                      ctypes.c_float, ctypes.c_void_p)


class KdaPrefillArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", _c_i32), ("num_heads", _c_i32), ("head_dim_k", _c_i32),
        ("head_dim_v", _c_i32), ("chunk_size", _c_i32), ("total_tokens", _c_i64),
        ("dtype", ctypes.c_int), ("flags", _c_u32), ("scale", _c_f32),
        ("gate_lower_bound", _c_f32),
        ("q", _p), ("k", _p), ("v", _p), ("gate", _p), ("beta", _p),
        ("conv_weight", _p), ("conv_bias", _p), ("conv_state_in", _p), ("conv_state_out", _p),
        ("state_in", _p), ("state_out", _p), ("o", _p), ("cu_seqlens", _p),
        ("cu_seqlens_host", _p), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
        ("state_slots", _p), ("num_slots", _c_i32), ("dv_tile", _c_i32), ("schedule", _c_i32),
    ]


# kda_schedule (include/kda.h); the automatic choice is the fused schedule from
# FUSED_MIN_PAIRS (sequence, head) pairs on (KDA_FUSED_MIN_PAIRS)
SCHEDULES = {"auto": 0, "one_pass": 1, "two_pass": 2, "fused": 3}
FUSED_MIN_PAIRS = 384


def _schedule_code(schedule):
    if isinstance(schedule, str):
        if schedule not in SCHEDULES:
            raise ValueError("schedule must be one of %s" % sorted(SCHEDULES))
        return SCHEDULES[schedule]
    return int(schedule)


class KdaDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", _c_i32), ("num_heads", _c_i32), ("head_dim_k", _c_i32),
        ("head_dim_v", _c_i32), ("dtype", ctypes.c_int), ("flags", _c_u32),
        ("scale", _c_f32), ("gate_lower_bound", _c_f32),
        ("q", _p), ("k", _p), ("v", _p), ("gate", _p), ("beta", _p),
        ("conv_weight", _p), ("conv_bias", _p), ("conv_state", _p), ("state", _p), ("o", _p),
        ("state_slots", _p), ("num_slots", _c_i32),
    ]


class KdaDecodeMultiArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", _c_i32), ("num_heads", _c_i32), ("head_dim_k", _c_i32),
        ("head_dim_v", _c_i32), ("num_tokens", _c_i32), ("dtype", ctypes.c_int),
        ("flags", _c_u32), ("scale", _c_f32), ("gate_lower_bound", _c_f32),
        ("q", _p), ("k", _p), ("v", _p), ("gate", _p), ("beta", _p),
        ("conv_weight", _p), ("conv_bias", _p), ("conv_state", _p), ("state", _p), ("o", _p),
        ("updates", _p), ("pending_updates", _p), ("pending_accepted", _p),
        ("pending_tokens", _c_i32), ("state_slots", _p), ("num_slots", _c_i32),
    ]


class KdaDecodeCommitArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", _c_i32), ("num_heads", _c_i32), ("head_dim_k", _c_i32),
        ("head_dim_v", _c_i32), ("num_tokens", _c_i32), ("dtype", ctypes.c_int),
        ("flags", _c_u32), ("accepted", _p), ("updates", _p), ("conv_state", _p), ("state", _p),
        ("state_slots", _p), ("num_slots", _c_i32),
    ]


class KdaStateCopyArgs(ctypes.Structure):
    _fields_ = [
        ("count", _c_i32), ("num_heads", _c_i32), ("head_dim_k", _c_i32), ("head_dim_v", _c_i32),
        ("num_slots", _c_i32), ("dtype", ctypes.c_int), ("flags", _c_u32),
        ("src_slots", _p), ("dst_slots", _p), ("state_src", _p), ("state_dst", _p),
        ("conv_src", _p), ("conv_dst", _p),
    ]


class KdaGateBetaArgs(ctypes.Structure):
    _fields_ = [
        ("total_tokens", _c_i64), ("hidden", _c_i32), ("rank", _c_i32), ("num_heads", _c_i32),
        ("head_dim_k", _c_i32), ("flags", _c_u32), ("gate_lower_bound", _c_f32),
        ("x", _p), ("w_a", _p), ("w_b", _p), ("w_beta", _p), ("gate", _p), ("beta", _p),
        ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
    ]


class KdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (status, msg))
        self.status = status


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkda.so (raises if it was not built) and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libkda.so not found at %s: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
        lib = ctypes.CDLL(path)
        lib.kda_abi_version.restype = ctypes.c_int
        lib.kda_set_spin_limit.restype = _c_i32
        lib.kda_set_spin_limit.argtypes = [_c_i32]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]  # kda_status (an int-sized enum)
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_short_conv.restype = ctypes.c_int
        lib.kda_short_conv.argtypes = [_p, _p, _c_i64, _c_i32, _p, _p, _p, _p, _p, _p, _c_i32,
                                       ctypes.c_int, _c_u32, _p]
        for f in ("kda_prefill", "kda_prefill_noalloc"):
            getattr(lib, f).restype = ctypes.c_int
            getattr(lib, f).argtypes = [ctypes.POINTER(KdaPrefillArgs), _p]
        for f in ("kda_prefill_workspace_size", "kda_prefill_workspace_full_size",
                  "kda_prefill_workspace_min_size"):
            getattr(lib, f).restype = ctypes.c_size_t
            getattr(lib, f).argtypes = [ctypes.POINTER(KdaPrefillArgs)]
        lib.kda_decode.restype = ctypes.c_int
        lib.kda_decode.argtypes = [ctypes.POINTER(KdaDecodeArgs), _p]
        lib.kda_decode_multi.restype = ctypes.c_int
        lib.kda_decode_multi.argtypes = [ctypes.POINTER(KdaDecodeMultiArgs), _p]
        lib.kda_decode_commit.restype = ctypes.c_int
        lib.kda_decode_commit.argtypes = [ctypes.POINTER(KdaDecodeCommitArgs), _p]
        lib.kda_gate_beta_proj.restype = ctypes.c_int
        lib.kda_gate_beta_proj.argtypes = [ctypes.POINTER(KdaGateBetaArgs), _p]
        lib.kda_gate_beta_workspace_size.restype = ctypes.c_size_t
        lib.kda_gate_beta_workspace_size.argtypes = [ctypes.POINTER(KdaGateBetaArgs)]
        lib.kda_state_copy.restype = ctypes.c_int
        lib.kda_state_copy.argtypes = [ctypes.POINTER(KdaStateCopyArgs), _p]
        if path == LIB_PATH:
            _lib = lib
        return lib


def _check(lib, status):
    if status != KDA_OK:
        raise KdaError(lib.kda_status_string(status).decode(), lib.kda_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _state_flag(state):
    """KDA_F_STATE_BF16 for a bf16 state tensor, 0 for fp32 (decode entry points)."""
    if state.dtype == torch.bfloat16:
        return KDA_F_STATE_BF16
    if state.dtype == torch.float32:
        return 0
    raise TypeError("state must be float32 or bfloat16, got %s" % state.dtype)


def _slots(state_slots, pools, n, dev):
    """(pointer, num_slots) of an optional int32 slot map.  `pools` are the state and
    conv-state tensors the map indexes: all of them must have the same number of
    rows (their first dimension), which becomes num_slots.  Without a map, each
    given pool must have one row per sequence."""
    pools = [t for t in pools if torch.is_tensor(t)]
    rows = {int(t.shape[0]) for t in pools}
    if state_slots is None:
        if rows and rows != {n}:
            raise ValueError("without state_slots, state and conv-state tensors need one row "
                             "per sequence (%d)" % n)
        return None, 0
    _need(state_slots, "state_slots", torch.int32, dev)
    if state_slots.numel() != n:
        raise ValueError("state_slots must hold one slot per sequence")
    if len(rows) != 1:
        raise ValueError("the state and conv-state pools must have the same number of rows")
    return _ptr(state_slots), rows.pop()


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s" % (name, device))


def _shape(t, name, shape):
    """Raise ValueError unless tensor `t` (if given) has exactly `shape`."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(int(x) for x in shape),
                                                            tuple(t.shape)))


def _conv_weight_shape(t, name, channels):
    """Conv weights hold 4 taps per channel: [channels, 4], or [3, channels / 3, 4]."""
    if t is None:
        return
    if t.numel() != channels * 4 or t.shape[-1] != 4:
        raise ValueError("%s must hold %d channels x 4 taps, got shape %s" % (name, channels,
                                                                             tuple(t.shape)))


def _pool_shape(t, name, rows_shape_tail):
    """A state or conv-state pool: any number of rows of the given trailing shape."""
    if t is not None and (t.dim() != 1 + len(rows_shape_tail) or
                          tuple(t.shape[1:]) != tuple(rows_shape_tail)):
        raise ValueError("%s must have shape [rows, %s], got %s" % (
            name, ", ".join(str(x) for x in rows_shape_tail), tuple(t.shape)))


def abi_version():
    return load_library().kda_abi_version()


def set_spin_limit(polls):
    """Bound of the fused prefill's hand-over waits, for tests of its failure path
    (kda_set_spin_limit): after `polls` unsuccessful polls a wait gives up and the
    call ends with wrong results instead of hanging.  polls <= 0 restores the
    default.  Returns the previous bound."""
    return load_library().kda_set_spin_limit(int(polls))


def kda_short_conv(x, weight, *, cu_seqlens=None, cu_seqlens_host=None, bias=None,
                   conv_state_in=None, conv_state_out=None, y=None, num_seqs=None, silu=False,
                   stream=None):
    """Causal depthwise conv, width 4.  x: [T, C] bf16/fp32 on the GPU; weight [C, 4] fp32.

    Returns y (allocated when not given).  conv_state_out=True allocates [N, 3, C]."""
    lib = load_library()
    dev = x.device
    if x.dim() != 2:
        raise ValueError("x must be [T, C], got %s" % (tuple(x.shape),))
    T, C = x.shape
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else int(num_seqs or 1)
    if y is None:
        y = torch.empty_like(x)
    if conv_state_out is True:
        conv_state_out = torch.empty((N, 3, C), dtype=x.dtype, device=dev)
    _shape(y, "y", (T, C))
    _shape(weight, "weight", (C, 4))
    _shape(bias, "bias", (C,))
    _shape(conv_state_in, "conv_state_in", (N, 3, C))
    _shape(conv_state_out, "conv_state_out", (N, 3, C))
    _shape(cu_seqlens, "cu_seqlens", (N + 1,))
    for t, nm in ((x, "x"), (y, "y"), (conv_state_in, "conv_state_in"),
                  (conv_state_out, "conv_state_out")):
        _need(t, nm, x.dtype, dev)
    _need(weight, "weight", torch.float32, dev)
    _need(bias, "bias", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    cuh = None
    if cu_seqlens_host is not None:
        cuh = cu_seqlens_host.to(torch.int32).contiguous().cpu()
    st = lib.kda_short_conv(_ptr(x), _ptr(y), T, C, _ptr(weight), _ptr(bias), _ptr(conv_state_in),
                            _ptr(conv_state_out), _ptr(cu_seqlens), _ptr(cuh), N, _dtype_code(x),
                            KDA_F_SILU if silu else 0, _stream(stream, dev))
    _check(lib, st)
    if conv_state_out is not None:
        return y, conv_state_out
    return y


def kda_prefill(q, k, v, gate, beta, conv_weight, *, cu_seqlens=None, cu_seqlens_host=None,
                num_seqs=None, conv_bias=None, conv_state_in=None, conv_state_out=None,
                state_in=None, state_out=None, o=None, scale=0.0, gate_lower_bound=-5.0,
                chunk_size=0, flags=0, workspace=True, state_slots=None, dv_tile=0, schedule="auto",
                stream=None, _entry="kda_prefill"):
    """Chunked KDA prefill of packed sequences (kda_prefill).

    The state (state_in / state_out) is fp32, or bf16 storage when those tensors are
    bf16 (state_out=True allocates the dtype of state_in, else fp32).  With
    state_slots (int32 [N]) the state and conv-state tensors are pools and sequence n
    uses row state_slots[n] (state_out / conv_state_out must then be given).

    q, k, gate: [T, H, 128]; v: [T, H, 128]; beta: [T, H] (bf16 or fp32, one dtype);
    conv_weight: [3*H*128, 4] fp32.  state_out / conv_state_out: a tensor, or True
    to allocate one.  schedule: "auto" (the library's choice), "one_pass",
    "two_pass" or "fused" (include/kda.h).  workspace: True (the default)
    allocates the two-pass workspace when the call will run that schedule; a
    uint8 device tensor is used as that workspace; None or False gives none (the
    automatic choice then runs the fused or the one-pass schedule).  dv_tile:
    state columns per workgroup (0 = automatic).  Returns (o, state_out,
    conv_state_out)."""
    lib = load_library()
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [T, H, 128], got %s" % (tuple(q.shape),))
    T, H, dk = q.shape
    dv = v.shape[-1] if v.dim() == 3 else -1
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else int(num_seqs or 1)
    CC = 2 * H * dk + H * dv
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if state_slots is not None and (state_out is True or conv_state_out is True):
        raise ValueError("with state_slots, pass the pool tensors as state_out / conv_state_out")
    if state_out is True:
        sdt = state_in.dtype if state_in is not None else torch.float32
        state_out = torch.empty((N, H, dk, dv), dtype=sdt, device=dev)
    if conv_state_out is True:
        conv_state_out = torch.empty((N, 3, CC), dtype=q.dtype, device=dev)
    for t, nm in ((k, "k"), (gate, "gate")):
        _shape(t, nm, (T, H, dk))
    _shape(v, "v", (T, H, dv))
    _shape(o, "o", (T, H, dv))
    _shape(beta, "beta", (T, H))
    _conv_weight_shape(conv_weight, "conv_weight", CC)
    _shape(conv_bias, "conv_bias", (CC,))
    _shape(cu_seqlens, "cu_seqlens", (N + 1,))
    if state_slots is None:
        _shape(state_in, "state_in", (N, H, dk, dv))
        _shape(state_out, "state_out", (N, H, dk, dv))
        _shape(conv_state_in, "conv_state_in", (N, 3, CC))
        _shape(conv_state_out, "conv_state_out", (N, 3, CC))
    else:
        for t, nm in ((state_in, "state_in"), (state_out, "state_out")):
            _pool_shape(t, nm, (H, dk, dv))
        for t, nm in ((conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
            _pool_shape(t, nm, (3, CC))
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"), (o, "o"),
                  (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _need(t, nm, q.dtype, dev)
    for t, nm in ((conv_weight, "conv_weight"), (conv_bias, "conv_bias")):
        _need(t, nm, torch.float32, dev)
    sflag = 0
    for t, nm in ((state_in, "state_in"), (state_out, "state_out")):
        _need(t, nm, None, dev)
    if state_in is not None and state_out is not None and state_in.dtype != state_out.dtype:
        raise TypeError("state_in and state_out must have one dtype")
    for t in (state_in, state_out):
        if t is not None:
            sflag = _state_flag(t)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    cuh = None
    if cu_seqlens_host is not None:
        cuh = torch.as_tensor(cu_seqlens_host).to(torch.int32).contiguous().cpu()
        _shape(cuh, "cu_seqlens_host", (N + 1,))
    a = KdaPrefillArgs(
        num_seqs=N, num_heads=H, head_dim_k=dk, head_dim_v=dv, chunk_size=int(chunk_size),
        total_tokens=T, dtype=_dtype_code(q), flags=int(flags) | sflag, scale=float(scale),
        gate_lower_bound=float(gate_lower_bound),
        q=_ptr(q), k=_ptr(k), v=_ptr(v), gate=_ptr(gate), beta=_ptr(beta),
        conv_weight=_ptr(conv_weight), conv_bias=_ptr(conv_bias),
        conv_state_in=_ptr(conv_state_in), conv_state_out=_ptr(conv_state_out),
        state_in=_ptr(state_in), state_out=_ptr(state_out), o=_ptr(o),
        cu_seqlens=_ptr(cu_seqlens), cu_seqlens_host=_ptr(cuh), workspace=None, workspace_bytes=0,
        dv_tile=int(dv_tile), schedule=_schedule_code(schedule))
    pools = (state_in, state_out, conv_state_in, conv_state_out)
    if state_slots is not None and not any(torch.is_tensor(t) for t in pools):
        raise ValueError("state_slots needs a state or conv-state pool")
    a.state_slots, a.num_slots = _slots(state_slots, pools, N, dev)
    if workspace is True:
        need = lib.kda_prefill_workspace_size(ctypes.byref(a))
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    elif workspace is False:
        workspace = None
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel()
    _check(lib, getattr(lib, _entry)(ctypes.byref(a), _stream(stream, dev)))
    return o, state_out, conv_state_out


def kda_prefill_noalloc(q, k, v, gate, beta, conv_weight, **kw):
    """kda_prefill through the entry point that allocates nothing (kda_prefill_noalloc):
    the two-pass schedule runs in the library's per-GPU scratch.  Same arguments as
    kda_prefill except `workspace`; pass o, state_out and conv_state_out as tensors
    where the caller must not allocate either."""
    if "workspace" in kw:
        raise ValueError("kda_prefill_noalloc takes no workspace")
    return kda_prefill(q, k, v, gate, beta, conv_weight, workspace=None, _entry="kda_prefill_noalloc",
                       **kw)


def prefill_workspace_bytes(total_tokens, num_heads, num_seqs=1, dtype=torch.bfloat16,
                            chunk_size=0, cu_seqlens_host=None, which="recommended", schedule="auto"):
    """Workspace bytes of the two-pass prefill: the recommended size
    ("recommended": the whole call up to PREFILL_WORKSPACE_CAP, windows beyond; 0
    when the call will not run two passes), the whole call at once ("full") or
    the smallest accepted ("min"; both 0 when the dtype or chunk excludes the
    schedule)."""
    lib = load_library()
    a = KdaPrefillArgs(num_seqs=int(num_seqs), num_heads=int(num_heads), head_dim_k=128,
                       head_dim_v=128, chunk_size=int(chunk_size), total_tokens=int(total_tokens),
                       dtype=KDA_BF16 if dtype == torch.bfloat16 else KDA_F32,
                       schedule=_schedule_code(schedule))
    cuh = None
    if cu_seqlens_host is not None:
        cuh = torch.as_tensor(cu_seqlens_host).to(torch.int32).contiguous().cpu()
        a.cu_seqlens_host = _ptr(cuh)
    fn = {"recommended": lib.kda_prefill_workspace_size, "full": lib.kda_prefill_workspace_full_size,
          "min": lib.kda_prefill_workspace_min_size}[which]
    return int(fn(ctypes.byref(a)))


def kda_decode(q, k, v, gate, beta, conv_weight, conv_state, state, *, conv_bias=None, o=None,
               scale=0.0, gate_lower_bound=-5.0, flags=0, state_slots=None, stream=None):
    """One decode step: q, k, gate, v: [N, H, 128]; beta [N, H]; conv_state [N, 3, CC]
    and state [N, H, 128, 128] (fp32, or bf16 storage) are updated in place.
    Returns o [N, H, 128]."""
    lib = load_library()
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [N, H, 128], got %s" % (tuple(q.shape),))
    N, H, dk = q.shape
    dv = v.shape[-1] if v.dim() == 3 else -1
    CC = 2 * H * dk + H * dv
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    for t, nm in ((k, "k"), (gate, "gate")):
        _shape(t, nm, (N, H, dk))
    _shape(v, "v", (N, H, dv))
    _shape(o, "o", (N, H, dv))
    _shape(beta, "beta", (N, H))
    _conv_weight_shape(conv_weight, "conv_weight", CC)
    _shape(conv_bias, "conv_bias", (CC,))
    if state_slots is None:
        _shape(state, "state", (N, H, dk, dv))
        _shape(conv_state, "conv_state", (N, 3, CC))
    else:
        _pool_shape(state, "state", (H, dk, dv))
        _pool_shape(conv_state, "conv_state", (3, CC))
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"), (o, "o"),
                  (conv_state, "conv_state")):
        _need(t, nm, q.dtype, dev)
    for t, nm in ((conv_weight, "conv_weight"), (conv_bias, "conv_bias")):
        _need(t, nm, torch.float32, dev)
    _need(state, "state", None, dev)
    a = KdaDecodeArgs(
        num_seqs=N, num_heads=H, head_dim_k=dk, head_dim_v=dv, dtype=_dtype_code(q),
        flags=int(flags) | _state_flag(state), scale=float(scale), gate_lower_bound=float(gate_lower_bound),
        q=_ptr(q), k=_ptr(k), v=_ptr(v), gate=_ptr(gate), beta=_ptr(beta),
        conv_weight=_ptr(conv_weight), conv_bias=_ptr(conv_bias), conv_state=_ptr(conv_state),
        state=_ptr(state), o=_ptr(o))
    a.state_slots, a.num_slots = _slots(state_slots, (state, conv_state), N, dev)
    _check(lib, lib.kda_decode(ctypes.byref(a), _stream(stream, dev)))
    return o


def kda_decode_multi(q, k, v, gate, beta, conv_weight, conv_state, state, *, updates=None,
                     conv_bias=None, o=None, pending_updates=None, pending_accepted=None,
                     scale=0.0, gate_lower_bound=-5.0, flags=0, state_slots=None, stream=None):
    """Speculative decode of T tokens per sequence.  q, k, gate, v: [N, T, H, 128];
    beta [N, T, H].  conv_state [N, 3, CC] and state [N, H, 128, 128] fp32 are only
    read, unless pending_updates ([N, H, T', 768] fp32 records of a previous call) and
    pending_accepted ([N] int32) are given: that commit is applied to them first.
    Returns (o [N, T, H, 128], updates [N, H, T, 768] fp32)."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [N, T, H, 128], got %s" % (tuple(q.shape),))
    N, T, H, dk = q.shape
    dv = v.shape[-1] if v.dim() == 4 else -1
    CC = 2 * H * dk + H * dv
    if o is None:
        o = torch.empty((N, T, H, dv), dtype=q.dtype, device=dev)
    if updates is None:
        updates = torch.empty((N, H, T, UPDATE_FLOATS), dtype=torch.float32, device=dev)
    for t, nm in ((k, "k"), (gate, "gate")):
        _shape(t, nm, (N, T, H, dk))
    _shape(v, "v", (N, T, H, dv))
    _shape(o, "o", (N, T, H, dv))
    _shape(beta, "beta", (N, T, H))
    _conv_weight_shape(conv_weight, "conv_weight", CC)
    _shape(conv_bias, "conv_bias", (CC,))
    if state_slots is None:
        _shape(state, "state", (N, H, dk, dv))
        _shape(conv_state, "conv_state", (N, 3, CC))
    else:
        _pool_shape(state, "state", (H, dk, dv))
        _pool_shape(conv_state, "conv_state", (3, CC))
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"), (o, "o"),
                  (conv_state, "conv_state")):
        _need(t, nm, q.dtype, dev)
    for t, nm in ((conv_weight, "conv_weight"), (conv_bias, "conv_bias"),
                  (updates, "updates"), (pending_updates, "pending_updates")):
        _need(t, nm, torch.float32, dev)
    _need(state, "state", None, dev)
    _need(pending_accepted, "pending_accepted", torch.int32, dev)
    if updates.numel() != N * H * T * UPDATE_FLOATS:
        raise ValueError("updates must hold N*H*T*%d floats" % UPDATE_FLOATS)
    pt = 0
    if pending_updates is not None:
        pt = pending_updates.numel() // (N * H * UPDATE_FLOATS)
        if pending_updates.numel() != N * H * pt * UPDATE_FLOATS:
            raise ValueError("pending_updates must hold N*H*T'*%d floats" % UPDATE_FLOATS)
        if pending_accepted is None or pending_accepted.numel() != N:
            raise ValueError("pending_accepted must be an int32 tensor of N counts")
    a = KdaDecodeMultiArgs(
        num_seqs=N, num_heads=H, head_dim_k=dk, head_dim_v=dv, num_tokens=T,
        dtype=_dtype_code(q), flags=int(flags) | _state_flag(state), scale=float(scale),
        gate_lower_bound=float(gate_lower_bound),
        q=_ptr(q), k=_ptr(k), v=_ptr(v), gate=_ptr(gate), beta=_ptr(beta),
        conv_weight=_ptr(conv_weight), conv_bias=_ptr(conv_bias), conv_state=_ptr(conv_state),
        state=_ptr(state), o=_ptr(o), updates=_ptr(updates),
        pending_updates=_ptr(pending_updates), pending_accepted=_ptr(pending_accepted),
        pending_tokens=pt)
    a.state_slots, a.num_slots = _slots(state_slots, (state, conv_state), N, dev)
    _check(lib, lib.kda_decode_multi(ctypes.byref(a), _stream(stream, dev)))
    return o, updates


def kda_decode_commit(updates, accepted, conv_state, state, *, state_slots=None, stream=None):
    """Advance state [N, H, 128, 128] (fp32 or bf16) and conv_state [N, 3, CC] in place over the
    first accepted[n] tokens ([N] int32 on the device) recorded in updates
    ([N, H, T, 768] fp32, written by kda_decode_multi)."""
    lib = load_library()
    dev = state.device
    N = accepted.numel()
    if state.dim() != 4:
        raise ValueError("state must be [rows, H, 128, 128], got %s" % (tuple(state.shape),))
    H, dk, dv = state.shape[1:]
    CC = 2 * H * dk + H * dv
    if state_slots is None:
        _shape(state, "state", (N, H, dk, dv))
        _shape(conv_state, "conv_state", (N, 3, CC))
    else:
        _pool_shape(conv_state, "conv_state", (3, CC))
    T = updates.numel() // (N * H * UPDATE_FLOATS)
    if updates.numel() != N * H * T * UPDATE_FLOATS:
        raise ValueError("updates must hold N*H*T*%d floats" % UPDATE_FLOATS)
    _need(updates, "updates", torch.float32, dev)
    _need(state, "state", None, dev)
    _need(conv_state, "conv_state", None, dev)
    _need(accepted, "accepted", torch.int32, dev)
    if accepted.numel() != N:
        raise ValueError("accepted must hold N counts")
    a = KdaDecodeCommitArgs(num_seqs=N, num_heads=H, head_dim_k=dk, head_dim_v=dv,
                            num_tokens=T, dtype=_dtype_code(conv_state),
                            flags=_state_flag(state), accepted=_ptr(accepted),
                            updates=_ptr(updates), conv_state=_ptr(conv_state), state=_ptr(state))
    a.state_slots, a.num_slots = _slots(state_slots, (state, conv_state), N, dev)
    _check(lib, lib.kda_decode_commit(ctypes.byref(a), _stream(stream, dev)))


def kda_state_copy(state_pool, src_slots, dst_slots, *, conv_pool=None, dst_state_pool=None,
                   dst_conv_pool=None, stream=None):
    """Copy pool rows: state (and conv state) of slot src_slots[i] to dst_slots[i]
    (int32 device tensors).  The destination pools default to the source pools."""
    lib = load_library()
    dev = state_pool.device
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [rows, H, 128, 128], got %s" % (tuple(state_pool.shape),))
    P, H, dk, dv = state_pool.shape
    CC = 2 * H * dk + H * dv
    for t, nm in ((conv_pool, "conv_pool"), (dst_conv_pool, "dst_conv_pool")):
        _shape(t, nm, (P, 3, CC))
    dst_state_pool = state_pool if dst_state_pool is None else dst_state_pool
    if conv_pool is not None and dst_conv_pool is None:
        dst_conv_pool = conv_pool
    for t, nm in ((state_pool, "state_pool"), (dst_state_pool, "dst_state_pool"),
                  (conv_pool, "conv_pool"), (dst_conv_pool, "dst_conv_pool")):
        _need(t, nm, None, dev)
    for t, nm in ((src_slots, "src_slots"), (dst_slots, "dst_slots")):
        _need(t, nm, torch.int32, dev)
    if src_slots.numel() != dst_slots.numel():
        raise ValueError("src_slots and dst_slots must have one length")
    if dst_state_pool.shape != state_pool.shape or dst_state_pool.dtype != state_pool.dtype:
        raise ValueError("the state pools must match in shape and dtype")
    a = KdaStateCopyArgs(count=src_slots.numel(), num_heads=H, head_dim_k=dk, head_dim_v=dv,
                         num_slots=P, dtype=_dtype_code(conv_pool) if conv_pool is not None else KDA_BF16,
                         flags=_state_flag(state_pool), src_slots=_ptr(src_slots),
                         dst_slots=_ptr(dst_slots), state_src=_ptr(state_pool),
                         state_dst=_ptr(dst_state_pool), conv_src=_ptr(conv_pool),
                         conv_dst=_ptr(dst_conv_pool))
    _check(lib, lib.kda_state_copy(ctypes.byref(a), _stream(stream, dev)))


def kda_gate_beta_proj(x, w_a, w_b, w_beta, *, gate=None, beta=None, workspace=None, log=False,
                       gate_lower_bound=-5.0, stream=None):
    """Gate and beta in-projections: x [T, hidden], w_a [128, hidden], w_b [H*128, 128],
    w_beta [H, hidden], all bf16.  Returns (gate [T, H, 128], beta [T, H]); with log=True
    the gate is lb * sigmoid(a) (pass KDA_F_GATE_IS_LOG to the mixer), else a.
    workspace: a uint8 tensor of at least kda_gate_beta_workspace_size bytes, or None
    to allocate one."""
    lib = load_library()
    dev = x.device
    if x.dim() != 2 or w_beta.dim() != 2:
        raise ValueError("x must be [T, hidden] and w_beta [H, hidden]")
    T, hidden = x.shape
    H = w_beta.shape[0]
    R = w_a.shape[0] if w_a.dim() == 2 else -1
    _shape(w_a, "w_a", (R, hidden))
    _shape(w_b, "w_b", (H * 128, R))
    _shape(w_beta, "w_beta", (H, hidden))
    if gate is None:
        gate = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    if beta is None:
        beta = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _shape(gate, "gate", (T, H, 128))
    _shape(beta, "beta", (T, H))
    for t, nm in ((x, "x"), (w_a, "w_a"), (w_b, "w_b"), (w_beta, "w_beta"), (gate, "gate"),
                  (beta, "beta")):
        _need(t, nm, torch.bfloat16, dev)
    a = KdaGateBetaArgs(total_tokens=T, hidden=hidden, rank=w_a.shape[0], num_heads=H,
                        head_dim_k=128, flags=KDA_F_GATE_IS_LOG if log else 0,
                        gate_lower_bound=float(gate_lower_bound), x=_ptr(x), w_a=_ptr(w_a),
                        w_b=_ptr(w_b), w_beta=_ptr(w_beta), gate=_ptr(gate), beta=_ptr(beta))
    if workspace is None:
        need = lib.kda_gate_beta_workspace_size(ctypes.byref(a))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(lib, lib.kda_gate_beta_proj(ctypes.byref(a), _stream(stream, dev)))
    return gate, beta


def gate_beta_workspace_bytes(total_tokens, num_heads):
    """Workspace bytes kda_gate_beta_proj needs."""
    lib = load_library()
    a = KdaGateBetaArgs(total_tokens=int(total_tokens), num_heads=int(num_heads))
    return int(lib.kda_gate_beta_workspace_size(ctypes.byref(a)))


# ------------------------------------------------------------------ calibration
CALIB_PATH = os.path.join(_HERE, "libkda_calib.so")
CALIB_EXPORTS = ("kda_calib_state_rmw", "kda_calib_copy", "kda_calib_fill")
_calib = None


def load_calib_library(path: str = CALIB_PATH):
    """Load libkda_calib.so: the measurement-only streaming kernels of known bytes
    (include/kda_calib.h)."""
    global _calib
    with _lock:
        if _calib is not None and path == CALIB_PATH:
            return _calib
        if not os.path.exists(path):
            raise RuntimeError("libkda_calib.so not found at %s: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
        lib = ctypes.CDLL(path)
        lib.kda_calib_state_rmw.argtypes = [_p, _c_i64, _c_f32, _p]
        lib.kda_calib_copy.argtypes = [_p, _p, ctypes.c_size_t, _p]
        lib.kda_calib_fill.argtypes = [_p, ctypes.c_size_t, _c_f32, _p]
        for f in CALIB_EXPORTS:
            getattr(lib, f).restype = ctypes.c_int
        if path == CALIB_PATH:
            _calib = lib
        return lib


def _calib_check(st, what):
    if st != 0:
        raise RuntimeError("%s failed with status %d" % (what, st))


def calib_state_rmw(state, scale=1.0, stream=None):
    """Read-modify-write of fp32 [rows, 128, 128]-shaped states in place (decode's
    state stream without its arithmetic)."""
    _need(state, "state", torch.float32, state.device)
    if state.numel() % (128 * 128):
        raise ValueError("state must hold whole 128 x 128 fp32 states")
    _calib_check(load_calib_library().kda_calib_state_rmw(
        _ptr(state), state.numel() // (128 * 128), float(scale), _stream(stream, state.device)),
        "kda_calib_state_rmw")


def calib_copy(dst, src, stream=None):
    """dst = src (byte sizes equal, multiples of 16)."""
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("dst and src must have one byte size")
    _need(dst, "dst", None, dst.device)
    _need(src, "src", None, dst.device)
    _calib_check(load_calib_library().kda_calib_copy(
        _ptr(dst), _ptr(src), dst.numel() * dst.element_size(), _stream(stream, dst.device)),
        "kda_calib_copy")


def calib_fill(dst, value=0.0, stream=None):
    """Every fp32 value of dst set to `value`."""
    _need(dst, "dst", None, dst.device)
    _calib_check(load_calib_library().kda_calib_fill(
        _ptr(dst), dst.numel() * dst.element_size(), float(value), _stream(stream, dst.device)),
        "kda_calib_fill")
