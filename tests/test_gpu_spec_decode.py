"""GPU parity of speculative multi-token decode (kda_decode_multi + kda_decode_commit).

The oracle is the token-by-token fp64 prefill: T speculative tokens of a sequence
are a prefill of T tokens from the sequence's state and conv cache, and a commit
of `a` accepted tokens is that prefill over the first `a` of them.  Bars as for
every entry point: fp32 max-abs <= 1e-4; bf16 relative L2 <= 2e-2 per (sequence,
head).  A second, stricter property ties the path to single-token decode: the
outputs and the committed state equal those of `a` kda_decode calls to fp32
rounding (single-token decode spreads a state over 512 threads, the verify over
256, so the 128 rows of a column are added in a different grouping), and the
conv cache bit for bit."""
import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import (BF16_REL, assert_f32_close, seeded, slice_rel_errors,
                               state_rel_errors, to_np)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _flat(x):
    """[N, T, ...] -> [N*T, ...] (the packed prefill layout)."""
    return x.reshape((-1,) + tuple(x.shape[2:]))


def _oracle_prefix(d, counts, state, conv_state, t0=0, **kw):
    """Oracle prefill of tokens t0 .. t0+counts[n]-1 of every sequence n."""
    N = d["q"].shape[0]
    sel = [slice(t0, t0 + int(c)) for c in counts]
    cat = lambda x: torch.cat([x[n, sel[n]].cpu() for n in range(N)], 0)
    cu = np.concatenate([[0], np.cumsum([int(c) for c in counts])]).astype(np.int32)
    return oracle.prefill(cat(d["q"]), cat(d["k"]), cat(d["v"]), cat(d["gate"]), cat(d["beta"]),
                          d["conv_w"], cu, state_in=state, conv_state_in=conv_state, **kw)


def _check(x, ref, dtype, what):
    """x, ref: [..., 128] rows; fp32 max-abs, bf16 relative L2 per row group."""
    if dtype == torch.float32:
        assert_f32_close(x, ref, what)
    else:
        a, b = to_np(x).reshape(-1, 128), to_np(ref).reshape(-1, 128)
        e = np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-30)
        assert e.max() <= BF16_REL, "%s rel err %.3g" % (what, e.max())


def _check_state(st, ref, dtype, what):
    if dtype == torch.float32:
        assert_f32_close(st, ref, what)
    else:
        assert state_rel_errors(st, ref).max() <= BF16_REL, what


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("flags", [0, kda.KDA_F_SILU | kda.KDA_F_GATE_IS_LOG, kda.KDA_F_NO_QK_L2NORM])
@pytest.mark.parametrize("T", [1, 6, 8])
def test_multi_and_commit_match_oracle(dtype, flags, T):
    N, H = 7, 3
    d = KI.make_spec_decode(N, T, H, dtype=dtype, seed=31 + T, device=DEV)
    if flags & kda.KDA_F_GATE_IS_LOG:
        d["gate"] = (-6.0 * seeded(d["gate"].shape, 32, "rand")).to(dtype)
    bias = 0.1 * seeded(d["conv_w"].shape[0], 33)
    st0, cs0 = d["state"].clone(), d["conv_state"].clone()
    o, upd = kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"],
                                  d["conv_state"], d["state"], conv_bias=bias, flags=flags)
    torch.cuda.synchronize()
    # verification leaves the state and the conv cache untouched
    assert torch.equal(d["state"], st0) and torch.equal(d["conv_state"], cs0)
    ref = _oracle_prefix(d, [T] * N, st0.cpu(), cs0.cpu(), conv_b=bias.cpu(), flags=flags)
    _check(o, ref["o"].reshape(N, T, H, 128), dtype, "multi o")
    # rows 3..5 of the records hold the raw tokens exactly
    u = upd.view(N, H, T, 6, 128)
    for row, x in ((3, d["q"]), (4, d["k"]), (5, d["v"])):
        assert torch.equal(u[:, :, :, row], x.float().permute(0, 2, 1, 3))
    # commit accepted prefixes, including none, all and out-of-range counts
    acc = torch.tensor([0, 1, T, min(3, T), T + 4, -2, max(T - 1, 0)], dtype=torch.int32)
    kda.kda_decode_commit(upd, acc.to(DEV), d["conv_state"], d["state"])
    torch.cuda.synchronize()
    keep = acc.clamp(0, T)
    refc = _oracle_prefix(d, keep.tolist(), st0.cpu(), cs0.cpu(), conv_b=bias.cpu(), flags=flags)
    _check_state(d["state"], refc["state"], dtype, "committed state")
    np.testing.assert_array_equal(to_np(d["conv_state"]), refc["conv_state"])
    for n in (0, 5):  # nothing accepted: bit-identical
        assert torch.equal(d["state"][n], st0[n]) and torch.equal(d["conv_state"][n], cs0[n])


def _close_to_rounding(x, ref, dtype, what):
    """x equals ref up to the fp32 summation order of one reduction (and, for bf16
    outputs, the one rounding step that such a difference can flip)."""
    x, ref = x.float(), ref.float()
    tol = (2.0 ** -7 if dtype == torch.bfloat16 else 2e-6) * ref.abs() + 1e-6
    bad = (x - ref).abs() > tol
    assert not bad.any(), "%s: %d values differ beyond rounding, max %.3g" % (
        what, int(bad.sum()), float((x - ref).abs().max()))


@pytest.mark.parametrize("lb", [-5.0, -8.6, -14.0])
def test_multi_scaled_state_range(lb):
    """The verify step runs on the state scaled by the running decay product when
    T (-lb) log2(e) <= 100 (lb = -5 and, at the edge with c near 2^-99, -8.6) and
    on the plain state otherwise (-14); decays pushed to the bound (gate inputs of
    +8, sigmoid near 1) make c as small as the bound allows."""
    N, H, T = 4, 3, 8
    d = KI.make_spec_decode(N, T, H, dtype=torch.float32, seed=61, device=DEV)
    d["gate"] = (8.0 + seeded(d["gate"].shape, 62)).to(torch.float32)
    st0, cs0 = d["state"].clone(), d["conv_state"].clone()
    o, upd = kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"],
                                  d["conv_state"], d["state"], gate_lower_bound=lb)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(upd).all()
    ref = _oracle_prefix(d, [T] * N, st0.cpu(), cs0.cpu(), gate_lower_bound=lb)
    _check(o, ref["o"].reshape(N, T, H, 128), torch.float32, "multi o, lb %g" % lb)
    acc = torch.tensor([T, 5, 1, 0], dtype=torch.int32)
    kda.kda_decode_commit(upd, acc.to(DEV), d["conv_state"], d["state"])
    torch.cuda.synchronize()
    refc = _oracle_prefix(d, acc.tolist(), st0.cpu(), cs0.cpu(), gate_lower_bound=lb)
    _check_state(d["state"], refc["state"], torch.float32, "committed state, lb %g" % lb)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_multi_and_commit_equal_decode_steps(dtype):
    N, H, T = 5, 4, 6
    d = KI.make_spec_decode(N, T, H, dtype=dtype, seed=41, device=DEV)
    bias = 0.1 * seeded(d["conv_w"].shape[0], 42)
    flags = kda.KDA_F_SILU
    # T single-token decode steps, keeping every intermediate state
    st, cs = d["state"].clone(), d["conv_state"].clone()
    outs, states, convs = [], [st.clone()], [cs.clone()]
    for t in range(T):
        outs.append(kda.kda_decode(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                   d["v"][:, t].contiguous(), d["gate"][:, t].contiguous(),
                                   d["beta"][:, t].contiguous(), d["conv_w"], cs, st,
                                   conv_bias=bias, flags=flags))
        states.append(st.clone())
        convs.append(cs.clone())
    o, upd = kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"],
                                  d["conv_state"], d["state"], conv_bias=bias, flags=flags)
    acc = torch.tensor([1, 2, 4, 6, 3], dtype=torch.int32)
    kda.kda_decode_commit(upd, acc.to(DEV), d["conv_state"], d["state"])
    torch.cuda.synchronize()
    _close_to_rounding(o, torch.stack(outs, 1), dtype, "o")
    for n, a in enumerate(acc.tolist()):
        _close_to_rounding(d["state"][n], states[a][n], torch.float32, "state %d" % n)
        assert torch.equal(d["conv_state"][n], convs[a][n]), n


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_pending_commit(dtype):
    """Two speculative steps; the second applies the first's commit itself."""
    N, H, T1, T2 = 6, 3, 6, 4
    d1 = KI.make_spec_decode(N, T1, H, dtype=dtype, seed=51, device=DEV)
    d2 = KI.make_spec_decode(N, T2, H, dtype=dtype, seed=52, device=DEV)
    d2["conv_w"] = d1["conv_w"]
    st0, cs0 = d1["state"].clone(), d1["conv_state"].clone()
    acc1 = torch.tensor([1, 6, 3, 0, 5, 2], dtype=torch.int32, device=DEV)
    _, upd1 = kda.kda_decode_multi(d1["q"], d1["k"], d1["v"], d1["gate"], d1["beta"],
                                   d1["conv_w"], d1["conv_state"], d1["state"])
    # separate commit, then step two
    st_a, cs_a = st0.clone(), cs0.clone()
    kda.kda_decode_commit(upd1, acc1, cs_a, st_a)
    o_a, upd_a = kda.kda_decode_multi(d2["q"], d2["k"], d2["v"], d2["gate"], d2["beta"],
                                      d2["conv_w"], cs_a, st_a)
    # fused: step two commits step one first
    o_b, upd_b = kda.kda_decode_multi(d2["q"], d2["k"], d2["v"], d2["gate"], d2["beta"],
                                      d2["conv_w"], d1["conv_state"], d1["state"],
                                      pending_updates=upd1, pending_accepted=acc1)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(upd_a, upd_b)
    assert torch.equal(d1["state"], st_a) and torch.equal(d1["conv_state"], cs_a)
    # against the oracle: accepted prefix of step one, then all of step two
    a1 = acc1.cpu().tolist()
    cat = lambda x1, x2: torch.cat([torch.cat([x1[n, :a1[n]].cpu(), x2[n].cpu()], 0)
                                    for n in range(N)], 0)
    cu = np.concatenate([[0], np.cumsum([a + T2 for a in a1])]).astype(np.int32)
    ref = oracle.prefill(cat(d1["q"], d2["q"]), cat(d1["k"], d2["k"]), cat(d1["v"], d2["v"]),
                         cat(d1["gate"], d2["gate"]), cat(d1["beta"], d2["beta"]), d1["conv_w"],
                         cu, state_in=st0.cpu(), conv_state_in=cs0.cpu())
    ro = np.stack([ref["o"][cu[n + 1] - T2:cu[n + 1]] for n in range(N)])
    _check(o_b, ro, dtype, "step two o")


def test_commit_all_equals_prefill_chunks():
    """Accepting every token equals a bf16 prefill over them (one state layout for
    both); the bar is the bf16 one per (sequence, head), as both sides round
    differently (bf16 matrix-core operands in prefill, fp32 in decode)."""
    N, H, T = 4, 2, 8
    d = KI.make_spec_decode(N, T, H, seed=61, device=DEV)
    st0, cs0 = d["state"].clone(), d["conv_state"].clone()
    o, upd = kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"],
                                  d["conv_state"], d["state"])
    kda.kda_decode_commit(upd, torch.full((N,), T, dtype=torch.int32, device=DEV),
                          d["conv_state"], d["state"])
    cu = torch.arange(0, (N + 1) * T, T, dtype=torch.int32, device=DEV)
    po, pst, pcs = kda.kda_prefill(_flat(d["q"]), _flat(d["k"]), _flat(d["v"]), _flat(d["gate"]),
                                   _flat(d["beta"]), d["conv_w"], cu_seqlens=cu, state_in=st0,
                                   conv_state_in=cs0, state_out=True, conv_state_out=True)
    torch.cuda.synchronize()
    e = slice_rel_errors(_flat(o), po, cu.cpu().tolist(), H)
    assert e.max() <= BF16_REL, e.max()
    assert state_rel_errors(d["state"], pst).max() <= BF16_REL
    assert torch.equal(d["conv_state"], pcs)


def test_spec_workload_full_size_sampled():
    """256 sequences x 6 tokens x 64 heads, fused with the previous step's commit, as
    timed; the oracle checks sampled sequences."""
    d0 = KI.workload_inputs(5, device=DEV)
    d = KI.workload_inputs(5, device=DEV, seed=105)
    d["conv_w"] = d0["conv_w"]
    N, T = d0["q"].shape[:2]
    acc0 = KI.make_accepted(N, T, seed=5, device=DEV)
    st0, cs0 = d0["state"].clone(), d0["conv_state"].clone()
    _, upd0 = kda.kda_decode_multi(d0["q"], d0["k"], d0["v"], d0["gate"], d0["beta"],
                                   d0["conv_w"], d0["conv_state"], d0["state"])
    o, upd = kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d0["conv_w"],
                                  d0["conv_state"], d0["state"], pending_updates=upd0,
                                  pending_accepted=acc0)
    acc = KI.make_accepted(N, T, seed=6, device=DEV)
    kda.kda_decode_commit(upd, acc, d0["conv_state"], d0["state"])
    torch.cuda.synchronize()
    a0, a1 = acc0.cpu().tolist(), acc.cpu().tolist()
    for n in (0, 77, 255):
        sl = slice(n, n + 1)
        L = a0[n] + T
        cat = lambda x0, x1: torch.cat([x0[n, :a0[n]].cpu(), x1[n].cpu()], 0)
        ref = oracle.prefill(cat(d0["q"], d["q"]), cat(d0["k"], d["k"]), cat(d0["v"], d["v"]),
                             cat(d0["gate"], d["gate"]), cat(d0["beta"], d["beta"]), d0["conv_w"],
                             np.array([0, L], np.int32), state_in=st0[sl].cpu(),
                             conv_state_in=cs0[sl].cpu())
        _check(o[n], ref["o"][a0[n]:], torch.bfloat16, "o seq %d" % n)
        # state after both commits: a0 of step one, then a1 of step two
        L2 = a0[n] + a1[n]
        ref2 = oracle.prefill(cat(d0["q"], d["q"])[:L2], cat(d0["k"], d["k"])[:L2],
                              cat(d0["v"], d["v"])[:L2], cat(d0["gate"], d["gate"])[:L2],
                              cat(d0["beta"], d["beta"])[:L2], d0["conv_w"],
                              np.array([0, L2], np.int32), state_in=st0[sl].cpu(),
                              conv_state_in=cs0[sl].cpu())
        assert state_rel_errors(d0["state"][sl], ref2["state"]).max() <= BF16_REL, n
        np.testing.assert_array_equal(to_np(d0["conv_state"][sl]), ref2["conv_state"])


def test_multi_rejects_overlapping_records():
    d = KI.make_spec_decode(2, 4, 2, seed=71, device=DEV)
    _, upd = kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"],
                                  d["conv_state"], d["state"])
    acc = torch.ones(2, dtype=torch.int32, device=DEV)
    with pytest.raises(kda.KdaError):
        kda.kda_decode_multi(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"],
                             d["conv_state"], d["state"], updates=upd, pending_updates=upd,
                             pending_accepted=acc)


# ------------------------------------------------------------- bf16 state storage

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bf16_state_decode_is_fp32_decode_rounded(dtype):
    """From the same (bf16-representable) state, bf16 storage runs the same fp32
    arithmetic and rounds once when it stores: o is bit-identical and the state is
    the fp32 result rounded to nearest even."""
    d = KI.make_decode(5, 3, dtype=dtype, seed=81, device=DEV)
    st16 = d["state"].to(torch.bfloat16)
    st32 = st16.float()
    cs_a, cs_b = d["conv_state"].clone(), d["conv_state"].clone()
    args = (d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"])
    o32 = kda.kda_decode(*args, cs_a, st32)
    o16 = kda.kda_decode(*args, cs_b, st16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32)
    assert torch.equal(st16, st32.to(torch.bfloat16))
    assert torch.equal(cs_a, cs_b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bf16_state_multi_and_commit(dtype):
    N, H, T = 6, 3, 6
    d = KI.make_spec_decode(N, T, H, dtype=dtype, seed=82, device=DEV)
    st16 = d["state"].to(torch.bfloat16)
    st32 = st16.float()
    st_init = st32.cpu()
    cs_a, cs_b = d["conv_state"].clone(), d["conv_state"].clone()
    args = (d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"])
    o32, u32 = kda.kda_decode_multi(*args, cs_a, st32)
    o16, u16 = kda.kda_decode_multi(*args, cs_b, st16)
    acc = torch.tensor([0, 1, 2, 4, 6, 3], dtype=torch.int32, device=DEV)
    kda.kda_decode_commit(u32, acc, cs_a, st32)
    kda.kda_decode_commit(u16, acc, cs_b, st16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32) and torch.equal(u16, u32)
    assert torch.equal(st16, st32.to(torch.bfloat16))
    assert torch.equal(cs_a, cs_b)
    # and against the oracle over the kept prefix, from the rounded initial state
    ref = _oracle_prefix(d, acc.cpu().tolist(), st_init, d["conv_state"].cpu())
    assert state_rel_errors(st16, ref["state"]).max() <= BF16_REL


# Accuracy study of bf16 state storage: (gate pre-activation mean, decode steps,
# bound on the bf16-state error).  Row decays exp(-5 sigmoid(a)) are about 0.08,
# 0.8, 0.99, 0.998 and 0.9998; the last (a memory of thousands of tokens) is the
# case where one rounding per step no longer stays inside the 2e-2 bar, and its
# bound records the measured level (2.4e-2) rather than the bar.
# (gate pre-activation mean, decode steps).  Row decays exp(-5 sigmoid(a)) of about
# 0.08, 0.8, 0.99, 0.998 and 0.9998.  bf16 storage meets the bf16 bar (2e-2) while
# the decays stay below about 0.998; at 0.9998 (memories of thousands of tokens) it
# measured 2.4e-2: a documented limit of the flag (include/kda.h), kept as a
# strict expected failure of the bar and bounded by the level test below.
BF16_STATE_LIMIT = 3e-2
BF16_STATE_STUDY = [(0.0, 256), (-3.0, 256), (-6.0, 384), (-8.0, 2048),
                    pytest.param(-10.0, 2048, marks=pytest.mark.xfail(
                        strict=True, raises=AssertionError,
                        reason="known limit of bf16 state storage: row decays near 0.9998 "
                               "measure 2.4e-2 against the 2e-2 bar"))]


def _bf16_state_errors(gate_mean, L):
    """L decode steps with the state stored as fp32 and as bf16 between steps, against
    the fp64 oracle over the same tokens (relative L2 per (sequence, head), max).
    Returns (fp32-storage o error, bf16-storage o error, bf16 final-state error)."""
    N, H = 2, 4
    inp = KI.make_prefill(H, [L] * N, seed=90, device=DEV, gate_mean=gate_mean, state_std=0.1,
                          conv_cache_std=1.0)
    st0 = inp["state_in"].to(torch.bfloat16)
    view = lambda x: x.view(N, L, *x.shape[1:])
    q, k, v, g, b = (view(inp[n]) for n in ("q", "k", "v", "gate", "beta"))
    res = {}
    for sd in (torch.float32, torch.bfloat16):
        st, cs = st0.to(sd).clone(), inp["conv_state_in"].clone()
        outs = []
        for t in range(L):
            outs.append(kda.kda_decode(q[:, t].contiguous(), k[:, t].contiguous(),
                                       v[:, t].contiguous(), g[:, t].contiguous(),
                                       b[:, t].contiguous(), inp["conv_w"], cs, st))
        torch.cuda.synchronize()
        res[sd] = (torch.stack(outs, 1).reshape(N * L, H, 128), st)
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                         inp["cu_seqlens"], state_in=st0.float().cpu(),
                         conv_state_in=inp["conv_state_in"].cpu())
    cu = inp["cu_seqlens"].cpu().tolist()
    e32 = slice_rel_errors(res[torch.float32][0], ref["o"], cu, H).max()
    e16 = slice_rel_errors(res[torch.bfloat16][0], ref["o"], cu, H).max()
    s16 = state_rel_errors(res[torch.bfloat16][1], ref["state"]).max()
    return e32, e16, s16


@pytest.mark.parametrize("gate_mean,L", BF16_STATE_STUDY)
def test_bf16_state_long_decode_accuracy(gate_mean, L):
    e32, e16, s16 = _bf16_state_errors(gate_mean, L)
    assert e32 <= BF16_REL, e32
    assert e16 <= BF16_REL and s16 <= BF16_REL, (e16, s16)


def test_bf16_state_near_one_decay_level():
    """Where bf16 storage misses the bar (decays near 0.9998) its error stays at the
    measured level rather than growing: each rounding decays with the state."""
    e32, e16, s16 = _bf16_state_errors(-10.0, 2048)
    assert e32 <= BF16_REL, e32
    assert e16 <= BF16_STATE_LIMIT and s16 <= BF16_STATE_LIMIT, (e16, s16)


@pytest.mark.parametrize("dtype,kw", [(torch.bfloat16, {"workspace": True}),
                                      (torch.bfloat16, {"chunk_size": 64}),
                                      (torch.float32, {"chunk_size": 32})])
def test_bf16_state_prefill_is_fp32_prefill_rounded(dtype, kw):
    """Prefill with bf16 state_in/state_out: the same outputs as fp32 storage of the
    same (bf16-representable) initial state, and the final state rounded once."""
    inp = KI.make_prefill(3, [40, 1, 77], dtype=dtype, seed=84, device=DEV, state_std=0.1,
                          conv_cache_std=1.0)
    s16 = inp["state_in"].to(torch.bfloat16)
    common = dict(cu_seqlens=inp["cu_seqlens"], conv_state_in=inp["conv_state_in"], **kw)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"])
    o32, st32, _ = kda.kda_prefill(*args, state_in=s16.float(), state_out=True, **common)
    o16, st16, _ = kda.kda_prefill(*args, state_in=s16, state_out=True, **common)
    torch.cuda.synchronize()
    assert st16.dtype == torch.bfloat16
    assert torch.equal(o16, o32)
    assert torch.equal(st16, st32.to(torch.bfloat16))


def test_bf16_state_prefill_then_decode_matches_oracle():
    """Disaggregated use: a prefill hands its bf16 final state and conv state to bf16-state
    decode steps; the whole run against the oracle over the concatenated tokens."""
    H, L, Td = 4, [50, 23], 5
    N = len(L)
    inp = KI.make_prefill(H, [a + Td for a in L], seed=85, device=DEV, state_std=0.1,
                          conv_cache_std=1.0)
    s0 = inp["state_in"].to(torch.bfloat16)
    cu = inp["cu_seqlens"].cpu().tolist()
    pre = torch.cat([torch.arange(cu[n], cu[n] + L[n]) for n in range(N)]).to(DEV)
    cu_p = torch.tensor([0, L[0], L[0] + L[1]], dtype=torch.int32, device=DEV)
    pick = lambda x, idx: x.index_select(0, idx).contiguous()
    o_p, st, cs = kda.kda_prefill(*(pick(inp[n], pre) for n in ("q", "k", "v", "gate", "beta")),
                                  inp["conv_w"], cu_seqlens=cu_p, state_in=s0,
                                  conv_state_in=inp["conv_state_in"], state_out=True,
                                  conv_state_out=True, workspace=True)
    outs = []
    for t in range(Td):
        idx = torch.tensor([cu[n] + L[n] + t for n in range(N)], device=DEV)
        outs.append(kda.kda_decode(*(pick(inp[n], idx) for n in ("q", "k", "v", "gate", "beta")),
                                   inp["conv_w"], cs, st))
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                         inp["cu_seqlens"], state_in=s0.float().cpu(),
                         conv_state_in=inp["conv_state_in"].cpu())
    o = torch.empty_like(inp["v"])
    o[pre] = o_p
    for t in range(Td):
        o[torch.tensor([cu[n] + L[n] + t for n in range(N)], device=DEV)] = outs[t]
    assert slice_rel_errors(o, ref["o"], cu, H).max() <= BF16_REL
    assert state_rel_errors(st, ref["state"]).max() <= BF16_REL
    np.testing.assert_array_equal(to_np(cs), ref["conv_state"])
