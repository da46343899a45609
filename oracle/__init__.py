"""fp64 CPU oracle for the KDA sequence mixer -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  It shares no code with the HIP
library in ``gated_delta_rule_short_amd`` and never touches a GPU.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, a token-by-token
recurrence; see its header for the passages it follows and the readings it
takes).  This module only compiles it with gcc, marshals numpy arrays through
ctypes and upcasts inputs: every input is first rounded to its storage dtype by
the caller (bf16 inputs stay bf16-valued) and then converted to float64, so the
oracle sees exactly the values the GPU sees.

Parity status of each function:
  short_conv -- pinned (torch conv1d with groups=C, one-hot shift taps).
  prefill    -- pinned (closed forms: beta=0 decay, one-hot-key GLA, orthonormal
                retrieval, beta=1 q=k self-read; brute-force unrolled products
                for T<=8; L2 and gate limits).
  decode     -- pinned through prefill (same recurrence, length-one sequences)
                and the decode-steps == prefill composition.
  gate_beta_proj -- pinned (zero weights give the sigmoid midpoints exactly;
                a brute-force scalar loop on tiny shapes; selection weights give
                the closed form; the sign symmetry of the sigmoid).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None

SILU = 1
NO_QK_L2NORM = 2
GATE_IS_LOG = 4


def build(force: bool = True) -> str:
    """Compile kda_oracle.c into libkda_oracle.so with gcc (-O2, OpenMP, IEEE)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    d, i64, u32, i32 = ctypes.c_double, ctypes.c_int64, ctypes.c_uint, ctypes.c_int
    p = ctypes.c_void_p
    lib.kda_oracle_short_conv.argtypes = [p, p, i64, i64, p, p, p, p, p, i64, i32, i32]
    lib.kda_oracle_short_conv.restype = None
    lib.kda_oracle_prefill.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, p,
                                       p, p, p, d, d, u32, i32]
    lib.kda_oracle_prefill.restype = None
    lib.kda_oracle_decode.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, p,
                                      d, d, u32, i32]
    lib.kda_oracle_decode.restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(x):
    """Upcast (torch tensor or array-like) to a C-contiguous float64 numpy array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: go through float64 on the CPU
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def short_conv(x, weight, cu_seqlens, bias=None, conv_state_in=None, silu=False,
               nthreads=0):
    """Causal depthwise conv, width 4.  x: [T, C]; weight: [C, 4] (tap 3 = current).

    Returns (y [T, C], conv_state_out [N, 3, C]) as float64 arrays."""
    lib = _load()
    x = _f64(x)
    w = _f64(weight)
    b = _f64(bias)
    cs = _f64(conv_state_in)
    cu = _i32(cu_seqlens)
    T, C = x.shape
    N = cu.shape[0] - 1
    assert w.shape == (C, 4) and cu[-1] == T
    y = np.zeros((T, C), np.float64)
    cso = np.zeros((N, 3, C), np.float64)
    lib.kda_oracle_short_conv(_ptr(x), _ptr(y), T, C, _ptr(w), _ptr(b), _ptr(cs), _ptr(cso),
                              _ptr(cu), N, int(bool(silu)), int(nthreads))
    return y, cso


def prefill(q, k, v, gate, beta, conv_w, cu_seqlens, conv_b=None, conv_state_in=None,
            state_in=None, scale=None, gate_lower_bound=-5.0, flags=0, nthreads=0):
    """Token-by-token KDA over packed sequences (fp64).

    q, k, gate: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; conv_w: [2*H*dk + H*dv, 4]
    (a [3, H*d, 4] array is accepted when dk == dv); cu_seqlens: [N+1].
    Returns dict(o [T,H,dv], state [N,H,dk,dv], conv_state [N,3,CC])."""
    lib = _load()
    q, k, v, gate, beta = map(_f64, (q, k, v, gate, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    CC = 2 * H * dk + H * dv
    w = _f64(conv_w).reshape(CC, 4)
    b = None if conv_b is None else _f64(conv_b).reshape(CC)
    cs = None if conv_state_in is None else _f64(conv_state_in)
    cu = _i32(cu_seqlens)
    N = cu.shape[0] - 1
    assert cu[-1] == T and k.shape == q.shape and gate.shape == q.shape
    assert beta.shape == (T, H) and v.shape[:2] == (T, H)
    if cs is not None:
        cs = np.ascontiguousarray(cs.reshape(N, 3, CC))
    s_in = None if state_in is None else np.ascontiguousarray(_f64(state_in).reshape(N, H, dk, dv))
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((T, H, dv), np.float64)
    s_out = np.zeros((N, H, dk, dv), np.float64)
    cs_out = np.zeros((N, 3, CC), np.float64)
    lib.kda_oracle_prefill(N, H, dk, dv, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                           _ptr(beta), _ptr(w), _ptr(b), _ptr(cs), _ptr(cs_out), _ptr(s_in),
                           _ptr(s_out), _ptr(o), float(scale), float(gate_lower_bound),
                           int(flags), int(nthreads))
    return {"o": o, "state": s_out, "conv_state": cs_out}


def decode(q, k, v, gate, beta, conv_w, conv_state, state, conv_b=None, scale=None,
           gate_lower_bound=-5.0, flags=0, nthreads=0):
    """One decode step for N sequences.  q, k, gate: [N, H, dk]; v: [N, H, dv];
    beta: [N, H]; conv_state: [N, 3, CC]; state: [N, H, dk, dv].

    Returns dict(o, state, conv_state) -- new arrays; the inputs are not modified."""
    lib = _load()
    q, k, v, gate, beta = map(_f64, (q, k, v, gate, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    CC = 2 * H * dk + H * dv
    w = _f64(conv_w).reshape(CC, 4)
    b = None if conv_b is None else _f64(conv_b).reshape(CC)
    cs = np.array(_f64(conv_state).reshape(N, 3, CC), copy=True)
    st = np.array(_f64(state).reshape(N, H, dk, dv), copy=True)
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((N, H, dv), np.float64)
    lib.kda_oracle_decode(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                          _ptr(w), _ptr(b), _ptr(cs), _ptr(st), _ptr(o), float(scale),
                          float(gate_lower_bound), int(flags), int(nthreads))
    return {"o": o, "state": st, "conv_state": cs}


def gate_beta_proj(x, w_a, w_b, w_beta, num_heads, gate_lower_bound=-5.0, log=False):
    """The gate and beta in-projections in fp64 (numpy products as primitives).

    Follows "GLM-5.3-Flash Internals" (hidden width, the named two-factor gate
    projection) and "GLM-5.3-Flash im Detail", section "Sequenz-Mixing"
    (channel-wise gate with log-decay >= lb, one beta per head and token):
        a    = (x W_a^T) W_b^T      x [T][hidden], W_a [r][hidden], W_b [H*dk][r]
        gate = a, or lb * sigmoid(a) when `log`
        beta = sigmoid(x W_beta^T)  W_beta [H][hidden]
    Returns dict(gate [T][H][dk], beta [T][H], a [T][H*dk]).  The reading that the
    two factors multiply in this order, with no bias and no other activation, is
    recorded in the design notes."""
    x, w_a, w_b, w_beta = map(_f64, (x, w_a, w_b, w_beta))
    T = x.shape[0]
    z = x @ w_a.T
    a = z @ w_b.T
    sig = lambda u: 1.0 / (1.0 + np.exp(-u))
    gate = gate_lower_bound * sig(a) if log else a
    beta = sig(x @ w_beta.T)
    return {"gate": gate.reshape(T, num_heads, -1), "beta": beta, "a": a}
