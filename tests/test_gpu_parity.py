"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element
by element on the same seeded inputs, plus invariants the chunked method must
keep.  Bars: fp32 inputs max-abs <= 1e-4; bf16 inputs relative L2 <= 2e-2 per
(sequence, head) slice, for outputs and final states."""
import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import (BF16_REL, assert_bf16_close, assert_f32_close, head_conv_state,
                               head_conv_w, seeded, slice_rel_errors, state_rel_errors, to_np)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _oracle_prefill(inp, **kw):
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                          inp["cu_seqlens"], state_in=inp.get("state_in"),
                          conv_state_in=inp.get("conv_state_in"), **kw)


def _gpu_prefill(inp, **kw):
    # this module's default is the one-pass schedule; two-pass cases pass workspace=True
    kw.setdefault("workspace", None)
    o, st, cs = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                inp["conv_w"], cu_seqlens=inp["cu_seqlens"],
                                state_in=inp.get("state_in"),
                                conv_state_in=inp.get("conv_state_in"), state_out=True,
                                conv_state_out=True, **kw)
    torch.cuda.synchronize()
    return o, st, cs


# ------------------------------------------------------------------ short conv

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_short_conv_matches_oracle(dtype, silu, with_state):
    g = torch.Generator(device="cpu").manual_seed(3)
    lengths = [37, 0, 1, 2, 3, 100, 64, 5]
    C = 390  # not a multiple of the 512 channels a block covers
    cu = KI.cu_from_lengths(lengths)
    T = int(cu[-1])
    x = torch.randn(T, C, generator=g).to(dtype)
    w = torch.randn(C, 4, generator=g) * 0.5
    b = torch.randn(C, generator=g) * 0.1
    cs = torch.randn(len(lengths), 3, C, generator=g).to(dtype) if with_state else None
    y, cso = kda.kda_short_conv(x.to(DEV), w.to(DEV), cu_seqlens=cu.to(DEV), cu_seqlens_host=cu,
                                bias=b.to(DEV), conv_state_in=None if cs is None else cs.to(DEV),
                                conv_state_out=True, silu=silu)
    torch.cuda.synchronize()
    ref, ref_cs = oracle.short_conv(x, w, cu, bias=b, conv_state_in=cs, silu=silu)
    yn = to_np(y)
    if dtype == torch.float32:
        np.testing.assert_allclose(yn, ref, rtol=1e-5, atol=1e-5)
    else:  # one bf16 rounding of the fp32 result
        np.testing.assert_allclose(yn, ref, rtol=2 ** -7, atol=1e-6)
    # the conv state is a copy of raw tokens: exact
    np.testing.assert_array_equal(to_np(cso), ref_cs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_short_conv_vector_path_matches_oracle(dtype, silu, with_state):
    """Channels a multiple of 16 bytes: the 16-byte path, with runs that sit inside a
    sequence, runs that straddle sequence starts and ends, and a partial channel block."""
    g = torch.Generator(device="cpu").manual_seed(5)
    lengths = [37, 0, 1, 2, 3, 100, 64, 5, 40, 19]
    C = 520
    cu = KI.cu_from_lengths(lengths)
    T = int(cu[-1])
    x = torch.randn(T, C, generator=g).to(dtype)
    w = torch.randn(C, 4, generator=g) * 0.5
    b = torch.randn(C, generator=g) * 0.1
    cs = torch.randn(len(lengths), 3, C, generator=g).to(dtype) if with_state else None
    y, cso = kda.kda_short_conv(x.to(DEV), w.to(DEV), cu_seqlens=cu.to(DEV), cu_seqlens_host=cu,
                                bias=b.to(DEV), conv_state_in=None if cs is None else cs.to(DEV),
                                conv_state_out=True, silu=silu)
    torch.cuda.synchronize()
    ref, ref_cs = oracle.short_conv(x, w, cu, bias=b, conv_state_in=cs, silu=silu)
    if dtype == torch.float32:
        np.testing.assert_allclose(to_np(y), ref, rtol=1e-5, atol=1e-5)
    else:
        np.testing.assert_allclose(to_np(y), ref, rtol=2 ** -7, atol=1e-6)
    np.testing.assert_array_equal(to_np(cso), ref_cs)


def test_short_conv_vector_path_long_dense():
    """A long dense batch (3 sequences x 1000 tokens, 2048 channels): mostly full runs."""
    g = torch.Generator(device="cpu").manual_seed(6)
    N, L, C = 3, 1000, 2048
    x = torch.randn(N * L, C, generator=g).to(torch.bfloat16)
    w = torch.randn(C, 4, generator=g) * 0.5
    ref, _ = oracle.short_conv(x, w, KI.cu_from_lengths([L] * N))
    y = kda.kda_short_conv(x.to(DEV), w.to(DEV), num_seqs=N)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(y), ref, rtol=2 ** -7, atol=1e-6)


def test_short_conv_dense_odd_channels_and_in_place_state():
    g = torch.Generator(device="cpu").manual_seed(4)
    N, L, C = 3, 21, 33
    x = torch.randn(N * L, C, generator=g)
    w = torch.randn(C, 4, generator=g)
    cs = torch.randn(N, 3, C, generator=g)
    ref, ref_cs = oracle.short_conv(x, w, KI.cu_from_lengths([L] * N), conv_state_in=cs)
    csd = cs.to(DEV)
    y = kda.kda_short_conv(x.to(DEV), w.to(DEV), num_seqs=N, conv_state_in=csd,
                           conv_state_out=csd)[0]
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(y), ref, rtol=1e-5, atol=1e-5)
    np.testing.assert_array_equal(to_np(csd), ref_cs)


# ---------------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("flags", [0, kda.KDA_F_SILU | kda.KDA_F_GATE_IS_LOG, kda.KDA_F_NO_QK_L2NORM])
def test_decode_matches_oracle(dtype, flags):
    d = KI.make_decode(6, 3, dtype=dtype, seed=21, device=DEV)
    if flags & kda.KDA_F_GATE_IS_LOG:
        d["gate"] = (-6.0 * seeded(d["gate"].shape, 22, "rand")).to(dtype)
    bias = 0.1 * seeded(d["conv_w"].shape[0], 23)
    ref = oracle.decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"], d["conv_state"],
                        d["state"], conv_b=bias, flags=flags)
    o = kda.kda_decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"], d["conv_state"],
                       d["state"], conv_bias=bias, flags=flags)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(d["conv_state"]), ref["conv_state"])
    if dtype == torch.float32:
        assert_f32_close(o, ref["o"], "decode o")
        assert_f32_close(d["state"], ref["state"], "decode state")
    else:
        e = np.linalg.norm((to_np(o) - ref["o"]).reshape(-1, 128), axis=1) / \
            np.linalg.norm(ref["o"].reshape(-1, 128), axis=1)
        assert e.max() <= BF16_REL
        assert state_rel_errors(d["state"], ref["state"]).max() <= BF16_REL


@pytest.mark.parametrize("chunk", [16, 32])
def test_prefill_tiny_fp32_max_abs(chunk):
    """The tiny fp32 workload (H=1, T=256): max-abs error <= 1e-4."""
    inp = KI.workload_inputs(0, device=DEV)
    ref = _oracle_prefill(inp)
    o, st, cs = _gpu_prefill(inp, chunk_size=chunk)
    assert_f32_close(o, ref["o"], "o")
    assert_f32_close(st, ref["state"], "state")
    np.testing.assert_array_equal(to_np(cs), ref["conv_state"])


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prefill_bf16_ragged(chunk):
    lengths = [1, 2, 3, 15, 16, 17, 0, 63, 64, 65, 130, 200]
    inp = KI.make_prefill(3, lengths, seed=31, device=DEV, state_std=0.1, conv_cache_std=1.0)
    ref = _oracle_prefill(inp)
    o, st, cs = _gpu_prefill(inp, chunk_size=chunk, cu_seqlens_host=inp["cu_seqlens"].cpu())
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 3, st, ref["state"], "chunk %d" % chunk)
    np.testing.assert_array_equal(to_np(cs), ref["conv_state"])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("flags", [kda.KDA_F_SILU, kda.KDA_F_NO_QK_L2NORM, kda.KDA_F_GATE_IS_LOG])
def test_prefill_flags_and_bias(dtype, flags):
    inp = KI.make_prefill(2, [40, 77], dtype=dtype, seed=41, device=DEV, state_std=0.1,
                          conv_cache_std=1.0)
    if flags & kda.KDA_F_GATE_IS_LOG:
        inp["gate"] = (-6.0 * seeded(inp["gate"].shape, 42, "rand")).to(dtype)
    if flags & kda.KDA_F_NO_QK_L2NORM:  # keep the delta rule contractive (beta |k|^2 < 1)
        inp["k"] = (0.5 * inp["k"].float()).to(dtype)
    bias = 0.1 * seeded(inp["conv_w"].shape[0], 43)
    ref = _oracle_prefill(inp, conv_b=bias, flags=flags, scale=0.3, gate_lower_bound=-4.0)
    o, st, cs = _gpu_prefill(inp, conv_bias=bias, flags=flags, scale=0.3, gate_lower_bound=-4.0)
    if dtype == torch.float32:
        assert_f32_close(o, ref["o"], "o")
        assert_f32_close(st, ref["state"], "state")
    else:
        assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 2, st, ref["state"])


@pytest.mark.parametrize("dv_tile", [32, 64, 128])
def test_prefill_dv_tiles_agree(dv_tile):
    inp = KI.make_prefill(2, [130, 70], seed=51, device=DEV, state_std=0.1)
    ref = _oracle_prefill(inp)
    o, st, _ = _gpu_prefill(inp, dv_tile=dv_tile)
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 2, st, ref["state"], "dv tile %d" % dv_tile)


def test_prefill_workload1_reduced_heads_full_length():
    """Single-sequence 4096-token prefill with 8 of the 64 heads, checked in full."""
    inp = KI.workload_inputs(1, device=DEV, H=8)
    ref = _oracle_prefill(inp)
    o, st, _ = _gpu_prefill(inp)
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 8, st, ref["state"])


def test_split_prefill_equals_whole():
    inp = KI.make_prefill(2, [300], seed=61, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _gpu_prefill(inp)
    for cut in (64, 100):
        a = {k_: (v_[:cut] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
        a["cu_seqlens"] = torch.tensor([0, cut], dtype=torch.int32, device=DEV)
        o1, st1, cs1 = _gpu_prefill(a)
        b = {k_: (v_[cut:] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
        b["cu_seqlens"] = torch.tensor([0, 300 - cut], dtype=torch.int32, device=DEV)
        b["state_in"], b["conv_state_in"] = st1, cs1
        o2, st2, cs2 = _gpu_prefill(b)
        e = slice_rel_errors(torch.cat([o1, o2]), o, [0, 300], 2)
        assert e.max() <= 1e-2
        assert state_rel_errors(st2, st).max() <= 1e-2
        assert torch.equal(cs2, cs)
        if cut % 64 == 0:  # chunk boundaries coincide: same arithmetic
            assert torch.equal(torch.cat([o1, o2]), o)


def test_prefill_equals_decode_steps():
    T = 9
    inp = KI.make_prefill(2, [T], seed=71, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _gpu_prefill(inp)
    state = inp["state_in"].clone()
    conv = inp["conv_state_in"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.kda_decode(inp["q"][t:t + 1], inp["k"][t:t + 1], inp["v"][t:t + 1],
                                   inp["gate"][t:t + 1], inp["beta"][t:t + 1], inp["conv_w"], conv,
                                   state))
    torch.cuda.synchronize()
    e = slice_rel_errors(torch.cat(outs), o, [0, T], 2)
    assert e.max() <= 1e-2
    assert state_rel_errors(state, st).max() <= 1e-2
    assert torch.equal(conv, cs)


def test_varlen_packed_equals_separate_calls_bitwise():
    lengths = [70, 0, 129, 5]
    inp = KI.make_prefill(2, lengths, seed=81, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _gpu_prefill(inp)
    cu = [int(c) for c in inp["cu_seqlens"]]
    for n, L in enumerate(lengths):
        a, b = cu[n], cu[n + 1]
        one = {k_: (v_[a:b] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
        one["cu_seqlens"] = torch.tensor([0, L], dtype=torch.int32, device=DEV)
        one["state_in"] = inp["state_in"][n:n + 1]
        one["conv_state_in"] = inp["conv_state_in"][n:n + 1]
        o1, st1, cs1 = _gpu_prefill(one)
        assert torch.equal(o1, o[a:b])
        assert torch.equal(st1, st[n:n + 1])
        assert torch.equal(cs1, cs[n:n + 1])
    # an empty sequence passes its states through
    assert torch.equal(st[1], inp["state_in"][1])
    assert torch.equal(cs[1], inp["conv_state_in"][1])


@pytest.mark.parametrize("workspace", [None, True])
def test_in_place_state_and_conv_state(workspace):
    inp = KI.make_prefill(2, [90, 33], seed=91, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _gpu_prefill(inp, workspace=workspace)
    s_io = inp["state_in"].clone()
    c_io = inp["conv_state_in"].clone()
    o2, _, _ = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                               inp["conv_w"], cu_seqlens=inp["cu_seqlens"], state_in=s_io,
                               state_out=s_io, conv_state_in=c_io, conv_state_out=c_io,
                               workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(s_io, st) and torch.equal(c_io, cs)


@pytest.mark.parametrize("workspace", [None, True])
def test_every_output_written_and_deterministic(workspace):
    inp = KI.make_prefill(3, [200, 1, 64], seed=101, device=DEV, state_std=0.1)
    T = inp["q"].shape[0]
    outs = []
    for _ in range(2):
        o = torch.full((T, 3, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        st = torch.full((3, 3, 128, 128), float("nan"), device=DEV)
        kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                        cu_seqlens=inp["cu_seqlens"], state_in=inp["state_in"], state_out=st, o=o,
                        workspace=workspace)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(st).any()
        outs.append((o, st))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_chunk_sizes_agree():
    inp = KI.make_prefill(2, [257], seed=111, device=DEV, state_std=0.1)
    res = [_gpu_prefill(inp, chunk_size=c) for c in (16, 32, 64)]
    for o, st, _ in res[1:]:
        assert slice_rel_errors(o, res[0][0], [0, 257], 2).max() <= 1e-2
        assert state_rel_errors(st, res[0][1]).max() <= 1e-2


@pytest.mark.parametrize("sched,kw,H,N", [("one_pass", {}, 1, 2), ("two_pass", {"workspace": True}, 1, 2),
                                         ("fused", {}, 1, 2), ("auto", {"workspace": True}, 64, 16)])
def test_empty_batch_and_zero_tokens(sched, kw, H, N):
    """No tokens at all: every schedule (the automatic one at 1024 pairs picks the
    fused kernel) returns an empty o and passes the states through unchanged."""
    inp = KI.make_prefill(H, [0] * N, seed=5, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _gpu_prefill(inp, schedule=sched, **kw)
    assert o.numel() == 0
    assert torch.equal(st, inp["state_in"]) and torch.equal(cs, inp["conv_state_in"])


# ------------------------------------------------- two-pass schedule (workspace)

@pytest.mark.parametrize("flags", [0, kda.KDA_F_SILU, kda.KDA_F_NO_QK_L2NORM, kda.KDA_F_GATE_IS_LOG])
def test_two_pass_ragged_matches_oracle(flags):
    _two_pass_ragged(flags)


@pytest.mark.parametrize("dv_tile", [16, 128])
def test_two_pass_silu_on_every_pass_b_kernel(dv_tile):
    """The SiLU instance of the narrow (16 columns) and the wide pass B."""
    _two_pass_ragged(kda.KDA_F_SILU, dv_tile=dv_tile)


def _two_pass_ragged(flags, dv_tile=0):
    lengths = [1, 2, 3, 15, 16, 17, 0, 63, 64, 65, 130, 200]
    inp = KI.make_prefill(3, lengths, seed=131, device=DEV, state_std=0.1, conv_cache_std=1.0)
    if flags & kda.KDA_F_GATE_IS_LOG:
        inp["gate"] = (-6.0 * seeded(inp["gate"].shape, 132, "rand")).to(torch.bfloat16)
    if flags & kda.KDA_F_NO_QK_L2NORM:
        # without the L2 norm the caller scales k; keep beta |k|^2 < 1 so the delta
        # rule stays contractive and bf16 rounding does not grow along the sequence
        inp["k"] = (0.5 * inp["k"].float()).to(torch.bfloat16)
    bias = 0.1 * seeded(inp["conv_w"].shape[0], 133)
    ref = _oracle_prefill(inp, conv_b=bias, flags=flags)
    o, st, cs = _gpu_prefill(inp, conv_bias=bias, flags=flags, workspace=True, dv_tile=dv_tile)
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 3, st, ref["state"], "two-pass")
    np.testing.assert_array_equal(to_np(cs), ref["conv_state"])


@pytest.mark.parametrize("dv_tile", [16, 32, 64, 128])
def test_two_pass_dv_tiles_agree_bitwise(dv_tile):
    inp = KI.make_prefill(2, [130, 70], seed=141, device=DEV, state_std=0.1)
    ref = _oracle_prefill(inp)
    base = _gpu_prefill(inp, workspace=True)
    o, st, _ = _gpu_prefill(inp, workspace=True, dv_tile=dv_tile)
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 2, st, ref["state"], "dv tile %d" % dv_tile)
    assert torch.equal(o, base[0]) and torch.equal(st, base[1])


@pytest.mark.parametrize("schedule", [{"workspace": True}, {"chunk_size": 64}])
def test_near_degenerate_keys(schedule):
    """beta = 1, nearly parallel keys and a weak decay: the strictly lower Gram of a
    chunk is close to all ones, so the triangular inverse and the delta rule's
    cancellation (each write overwrites almost the same direction) are at their
    hardest; still within the bf16 bar of the oracle, on both schedules."""
    H, lengths = 2, [16, 47, 100]
    inp = KI.make_prefill(H, lengths, seed=171, device=DEV, state_std=0.1)
    T = sum(lengths)
    base = seeded((1, H, 128), 172)
    inp["k"] = (base + 0.05 * seeded((T, H, 128), 173)).to(torch.bfloat16)
    inp["beta"] = torch.ones((T, H), dtype=torch.bfloat16, device=DEV)
    inp["gate"] = torch.full((T, H, 128), -4.0, dtype=torch.bfloat16, device=DEV)
    ref = _oracle_prefill(inp)
    o, st, _ = _gpu_prefill(inp, **schedule)
    assert torch.isfinite(o).all() and torch.isfinite(st).all()
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], H, st, ref["state"], "near-degenerate keys")


def test_two_pass_agrees_with_one_pass_chunk16():
    inp = KI.make_prefill(2, [257, 40], seed=151, device=DEV, state_std=0.1)
    a = _gpu_prefill(inp, workspace=True)
    b = _gpu_prefill(inp, chunk_size=16)
    assert slice_rel_errors(a[0], b[0], inp["cu_seqlens"].cpu(), 2).max() <= 1e-2
    assert state_rel_errors(a[1], b[1]).max() <= 1e-2


def test_two_pass_split_equals_whole_and_deterministic():
    inp = KI.make_prefill(2, [300], seed=161, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _gpu_prefill(inp, workspace=True)
    o_again, st_again, _ = _gpu_prefill(inp, workspace=True)
    assert torch.equal(o, o_again) and torch.equal(st, st_again)
    cut = 112  # a multiple of 16: sub-chunk boundaries coincide
    a = {k_: (v_[:cut] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
    a["cu_seqlens"] = torch.tensor([0, cut], dtype=torch.int32, device=DEV)
    o1, st1, cs1 = _gpu_prefill(a, workspace=True)
    b = {k_: (v_[cut:] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
    b["cu_seqlens"] = torch.tensor([0, 300 - cut], dtype=torch.int32, device=DEV)
    b["state_in"], b["conv_state_in"] = st1, cs1
    o2, st2, cs2 = _gpu_prefill(b, workspace=True)
    assert torch.equal(torch.cat([o1, o2]), o) and torch.equal(st2, st) and torch.equal(cs2, cs)
