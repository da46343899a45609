"""Seeded synthetic inputs for the KDA mixer, shared by the tests, the smoke
check and the benchmark.

This module holds no arithmetic of the method itself: it only draws random
tensors with fixed shapes, distributions and draw order, and rounds them to
their storage dtype.  Both the HIP path and the oracle receive exactly these
tensors (the oracle gets float64 copies of the rounded values).

Workloads (H heads of dimension d = dk = dv = 128, the published head shape):
  0  tiny     : 1 sequence, H=1, T=256, fp32
  1  prefill  : 1 sequence, H=64, T=4096, bf16, zero initial state
  2  decode   : 256 sequences x 1 token, H=64, bf16 tokens, state ~ 0.1 N(0,1)
  3  long     : 1 sequence, H=64, T=65536, gate pre-activation ~ N(2,1)
  4  varlen   : 16 sequences, lengths ~ U{512..16384}, state ~ 0.1 N(0,1)
  5  spec     : 256 sequences x 6 speculative tokens (k = 5 drafts + 1), H=64,
                bf16 tokens, state ~ 0.1 N(0,1), conv cache; accepted counts
                1 + Binomial(5, 0.8) (about four of five drafts kept)

Draw recipe (torch.Generator on the target device, seeded with the workload's
seed, all draws fp32 standard normals unless stated), in this order:
  lengths (varlen only, integer uniform) -> q -> k (each (token, head) row
  scaled to a random unit direction) -> v -> conv weight (std 0.5) -> gate
  pre-activation a ~ N(gate_mean, 1) -> beta = logistic(N(0,1)) ->
  initial state (if any, std state_std) -> conv cache (if any, like q).
The logistic applied to beta's draw and the unit-direction scaling of k shape
the *input distribution*; the mixer's own conv, L2 normalisation and gate are
not computed here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

D = 128
H_MODEL = 64


@dataclass
class Workload:
    name: str
    kind: str                      # "prefill", "decode" or "spec_decode"
    H: int = H_MODEL
    T: int = 0                     # tokens per sequence (dense prefill)
    num_seqs: int = 1
    lengths: Optional[tuple] = None  # (lo, hi) uniform lengths for varlen
    dtype: torch.dtype = torch.bfloat16
    gate_mean: float = 0.0
    state_std: Optional[float] = None
    conv_cache: bool = False
    seed: int = 0
    chunk: int = 64
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload("tiny_fp32_T256_H1", "prefill", H=1, T=256, dtype=torch.float32, seed=0),
    1: Workload("prefill_bf16_B1_T4096_H64", "prefill", T=4096, seed=1),
    2: Workload("decode_bf16_N256_H64", "decode", num_seqs=256, state_std=0.1,
                conv_cache=True, seed=2),
    3: Workload("long_prefill_bf16_B1_T65536_H64", "prefill", T=65536, gate_mean=2.0, seed=3),
    4: Workload("varlen_prefill_bf16_N16_U512_16384_H64", "prefill", num_seqs=16,
                lengths=(512, 16384), state_std=0.1, seed=4),
    5: Workload("spec_decode_bf16_N256_T6_H64", "spec_decode", num_seqs=256, T=6,
                state_std=0.1, conv_cache=True, seed=5, extra={"accept_p": 0.8}),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(g, shape, device, std=1.0, mean=0.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x


def _unit_rows(x):
    """Scale every last-axis row to a unit direction (input distribution only)."""
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def make_lengths(num_seqs, lo, hi, seed, device="cpu"):
    g = _gen("cpu", seed)
    return torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()


def cu_from_lengths(lengths, device="cpu"):
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def make_prefill(H, lengths, dtype=torch.bfloat16, seed=0, device="cpu", gate_mean=0.0,
                 state_std=None, conv_cache_std=None, conv_w_std=0.5, dk=D, dv=D):
    """Packed prefill inputs for sequences of the given lengths.

    Returns a dict: q, k, v, gate, beta ([T, H, .] in `dtype`), conv_w ([2H dk + H dv, 4]
    fp32), cu_seqlens (int32), lengths (list), state_in ([N,H,dk,dv] fp32 or None),
    conv_state_in ([N,3,CC] in `dtype` or None)."""
    lengths = [int(L) for L in lengths]
    N = len(lengths)
    T = sum(lengths)
    g = _gen(device, seed)
    q = _randn(g, (T, H, dk), device)
    k = _unit_rows(_randn(g, (T, H, dk), device))
    v = _randn(g, (T, H, dv), device)
    CC = 2 * H * dk + H * dv
    conv_w = _randn(g, (CC, 4), device, std=conv_w_std)
    a = _randn(g, (T, H, dk), device, mean=gate_mean)
    beta = torch.sigmoid(_randn(g, (T, H), device))
    state = None
    if state_std is not None:
        state = _randn(g, (N, H, dk, dv), device, std=state_std)
    conv_state = None
    if conv_cache_std is not None:
        conv_state = _randn(g, (N, 3, CC), device, std=conv_cache_std).to(dtype)
    return {
        "q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype), "gate": a.to(dtype),
        "beta": beta.to(dtype), "conv_w": conv_w, "cu_seqlens": cu_from_lengths(lengths, device),
        "lengths": lengths, "state_in": state, "conv_state_in": conv_state,
        "H": H, "dk": dk, "dv": dv,
    }


def make_decode(N, H, dtype=torch.bfloat16, seed=2, device="cpu", state_std=0.1,
                conv_w_std=0.5, gate_mean=0.0, dk=D, dv=D):
    """One new token for each of N sequences, with a state and a conv cache."""
    g = _gen(device, seed)
    q = _randn(g, (N, H, dk), device)
    k = _unit_rows(_randn(g, (N, H, dk), device))
    v = _randn(g, (N, H, dv), device)
    CC = 2 * H * dk + H * dv
    conv_w = _randn(g, (CC, 4), device, std=conv_w_std)
    a = _randn(g, (N, H, dk), device, mean=gate_mean)
    beta = torch.sigmoid(_randn(g, (N, H), device))
    state = _randn(g, (N, H, dk, dv), device, std=state_std)
    conv_state = _randn(g, (N, 3, CC), device).to(dtype)
    return {
        "q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype), "gate": a.to(dtype),
        "beta": beta.to(dtype), "conv_w": conv_w, "state": state, "conv_state": conv_state,
        "H": H, "dk": dk, "dv": dv,
    }


def make_spec_decode(N, T, H, dtype=torch.bfloat16, seed=5, device="cpu", state_std=0.1,
                     conv_w_std=0.5, gate_mean=0.0, dk=D, dv=D):
    """T speculative tokens for each of N sequences ([N, T, H, .] layouts), with a
    state and a conv cache; draws in the order of make_decode."""
    g = _gen(device, seed)
    q = _randn(g, (N, T, H, dk), device)
    k = _unit_rows(_randn(g, (N, T, H, dk), device))
    v = _randn(g, (N, T, H, dv), device)
    CC = 2 * H * dk + H * dv
    conv_w = _randn(g, (CC, 4), device, std=conv_w_std)
    a = _randn(g, (N, T, H, dk), device, mean=gate_mean)
    beta = torch.sigmoid(_randn(g, (N, T, H), device))
    state = _randn(g, (N, H, dk, dv), device, std=state_std)
    conv_state = _randn(g, (N, 3, CC), device).to(dtype)
    return {
        "q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype), "gate": a.to(dtype),
        "beta": beta.to(dtype), "conv_w": conv_w, "state": state, "conv_state": conv_state,
        "H": H, "T": T, "dk": dk, "dv": dv,
    }


def make_accepted(N, T, seed, p=0.8, device="cpu"):
    """Accepted tokens per sequence of a speculative step: the first token always,
    then each of the T - 1 drafts with probability p (int32 [N], values 1..T)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    kept = (torch.rand((N, T - 1), generator=g) < p).sum(1) if T > 1 else torch.zeros(N)
    return (1 + kept).to(torch.int32).to(device)


def make_gate_proj(T, hidden=4096, H=H_MODEL, rank=128, seed=6, device="cpu", dk=D):
    """Hidden states and synthetic in-projection weights for the gate and beta
    projections: x ~ N(0, 1) (a normalised residual stream), W_a ~ N(0, 1/hidden),
    W_b ~ N(0, 1/rank), W_beta ~ N(0, 1/hidden), so the gate pre-activation and
    beta's argument are about N(0, 1), as in the mixer workloads.  All bf16."""
    g = _gen(device, seed)
    x = _randn(g, (T, hidden), device)
    w_a = _randn(g, (rank, hidden), device, std=hidden ** -0.5)
    w_b = _randn(g, (H * dk, rank), device, std=rank ** -0.5)
    w_beta = _randn(g, (H, hidden), device, std=hidden ** -0.5)
    bf = torch.bfloat16
    return {"x": x.to(bf), "w_a": w_a.to(bf), "w_b": w_b.to(bf), "w_beta": w_beta.to(bf), "H": H}


def workload_inputs(idx, device="cpu", H=None, T=None, num_seqs=None, seed=None):
    """Inputs of workload `idx`, optionally shrunk (fewer heads/tokens/sequences)
    with the same distributions, for parity cases the oracle finishes quickly."""
    w = WORKLOADS[idx]
    H = w.H if H is None else H
    seed = w.seed if seed is None else seed
    if w.kind == "spec_decode":
        N = w.num_seqs if num_seqs is None else num_seqs
        return make_spec_decode(N, w.T if T is None else T, H, dtype=w.dtype, seed=seed,
                                device=device, state_std=w.state_std, gate_mean=w.gate_mean)
    if w.kind == "decode":
        N = w.num_seqs if num_seqs is None else num_seqs
        return make_decode(N, H, dtype=w.dtype, seed=seed, device=device, state_std=w.state_std,
                           gate_mean=w.gate_mean)
    if w.lengths is not None:
        N = w.num_seqs if num_seqs is None else num_seqs
        lengths = make_lengths(N, w.lengths[0], w.lengths[1], seed)
        if T is not None:  # shrink every length proportionally, keeping raggedness
            tot = sum(lengths)
            lengths = [max(1, int(round(L * T / tot))) for L in lengths]
    else:
        lengths = [w.T if T is None else T] * (w.num_seqs if num_seqs is None else num_seqs)
    return make_prefill(H, lengths, dtype=w.dtype, seed=seed, device=device,
                        gate_mean=w.gate_mean, state_std=w.state_std)


def bytes_per_token_head(dtype_bytes=2, dk=D, dv=D):
    """Algorithmic HBM bytes per (token, head) of prefill: q, k, v, gate, beta in,
    o out (the state and conv tails are per sequence)."""
    return dtype_bytes * (2 * dk + dv + dk + 1 + dv)


def prefill_flops_per_token_head(C=64, dk=D, dv=D):
    """Algorithmic MFMA FLOPs per (token, head) of the chunked form with 16-row
    blocks: the block-lower C x C Grams (A, P) and W (10 of 16 blocks for C=64),
    U0 = T V and P U, plus the three state contractions (W S, Qg S, Kd^T U).
    For C=64, d=128 this is 149,504."""
    nb = C // 16
    lower = (nb * (nb + 1) // 2) / (nb * nb)
    return 2 * (3 * lower * C * dk + 2 * lower * C * dv + 3 * dk * dv)


__all__ = ["WORKLOADS", "Workload", "make_prefill", "make_decode", "make_spec_decode",
           "make_accepted", "make_gate_proj", "workload_inputs",
           "make_lengths", "cu_from_lengths", "bytes_per_token_head",
           "prefill_flops_per_token_head", "D", "H_MODEL"]
