"""The fused prefill schedule (one workgroup per (sequence, head): the 16-token
operands are formed in LDS while the state is carried over them) against the
fp64 oracle, on ragged lengths and every flag, and the properties the other
schedules keep: bf16 state storage equals fp32 storage rounded once, pool slots
equal gathered rows, in-place state, a split sequence equals the whole one bit for
bit, determinism, and the automatic choice for many pairs."""
import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import BF16_REL, assert_bf16_close, seeded, state_rel_errors, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _oracle(inp, **kw):
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                          inp["cu_seqlens"], state_in=inp.get("state_in"),
                          conv_state_in=inp.get("conv_state_in"), **kw)


def _fused(inp, **kw):
    kw.setdefault("schedule", "fused")
    kw.setdefault("state_out", True)
    kw.setdefault("conv_state_out", True)
    o, st, cs = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                inp["conv_w"], cu_seqlens=inp["cu_seqlens"],
                                state_in=inp.get("state_in"),
                                conv_state_in=inp.get("conv_state_in"), **kw)
    torch.cuda.synchronize()
    return o, st, cs


LENGTHS = [1, 2, 3, 15, 16, 17, 0, 63, 64, 65, 130, 200, 1000]


@pytest.mark.parametrize("flags", [0, kda.KDA_F_SILU, kda.KDA_F_NO_QK_L2NORM, kda.KDA_F_GATE_IS_LOG])
def test_fused_ragged_matches_oracle(flags):
    inp = KI.make_prefill(3, LENGTHS, seed=231, device=DEV, state_std=0.1, conv_cache_std=1.0)
    if flags & kda.KDA_F_GATE_IS_LOG:
        inp["gate"] = (-6.0 * seeded(inp["gate"].shape, 232, "rand")).to(torch.bfloat16)
    if flags & kda.KDA_F_NO_QK_L2NORM:
        # without the L2 norm the caller scales k (beta |k|^2 < 1 keeps the delta rule
        # contractive, so bf16 rounding does not grow along the sequence)
        inp["k"] = (0.5 * inp["k"].float()).to(torch.bfloat16)
    bias = 0.1 * seeded(inp["conv_w"].shape[0], 233)
    ref = _oracle(inp, conv_b=bias, flags=flags)
    o, st, cs = _fused(inp, conv_bias=bias, flags=flags)
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], 3, st, ref["state"], "fused")
    np.testing.assert_array_equal(to_np(cs), ref["conv_state"])


def test_fused_without_initial_state_and_near_degenerate_keys():
    """No initial state or conv cache (zeros); then beta = 1 with nearly parallel
    keys and a weak decay, where the triangular inverse is hardest."""
    H, lengths = 2, [16, 47, 100, 333]
    inp = KI.make_prefill(H, lengths, seed=241, device=DEV)
    inp.pop("state_in", None)
    inp.pop("conv_state_in", None)
    ref = _oracle(inp)
    o, st, _ = _fused(inp)
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], H, st, ref["state"], "zero initial state")
    T = sum(lengths)
    base = seeded((1, H, 128), 242)
    inp["k"] = (base + 0.05 * seeded((T, H, 128), 243)).to(torch.bfloat16)
    inp["beta"] = torch.ones((T, H), dtype=torch.bfloat16, device=DEV)
    inp["gate"] = torch.full((T, H, 128), -4.0, dtype=torch.bfloat16, device=DEV)
    ref = _oracle(inp)
    o, st, _ = _fused(inp)
    assert torch.isfinite(o).all() and torch.isfinite(st).all()
    assert_bf16_close(o, ref["o"], inp["cu_seqlens"], H, st, ref["state"], "near-degenerate keys")


def test_fused_split_equals_whole_in_place_and_deterministic():
    inp = KI.make_prefill(2, [300], seed=251, device=DEV, state_std=0.1, conv_cache_std=1.0)
    o, st, cs = _fused(inp)
    o2, st2, cs2 = _fused(inp)
    assert torch.equal(o, o2) and torch.equal(st, st2) and torch.equal(cs, cs2)
    cut = 112  # a multiple of 16: sub-chunk boundaries coincide
    a = {k_: (v_[:cut] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
    a["cu_seqlens"] = torch.tensor([0, cut], dtype=torch.int32, device=DEV)
    oa, sta, csa = _fused(a)
    b = {k_: (v_[cut:] if k_ in ("q", "k", "v", "gate", "beta") else v_) for k_, v_ in inp.items()}
    b["cu_seqlens"] = torch.tensor([0, 300 - cut], dtype=torch.int32, device=DEV)
    b["state_in"], b["conv_state_in"] = sta, csa
    ob, stb, csb = _fused(b)
    assert torch.equal(torch.cat([oa, ob]), o) and torch.equal(stb, st) and torch.equal(csb, cs)
    # in place: state_out = state_in, conv_state_out = conv_state_in
    s_io = inp["state_in"].clone()
    c_io = inp["conv_state_in"].clone()
    inp2 = dict(inp, state_in=s_io, conv_state_in=c_io)
    o3, _, _ = _fused(inp2, state_out=s_io, conv_state_out=c_io)
    assert torch.equal(o3, o) and torch.equal(s_io, st) and torch.equal(c_io, cs)


def test_fused_bf16_state_and_pool_slots():
    """bf16 state storage equals fp32 storage of the same state rounded once at the
    end; pool slots map each sequence to its rows and leave the others alone."""
    H, lengths = 2, [70, 0, 33, 160]
    inp = KI.make_prefill(H, lengths, seed=261, device=DEV, state_std=0.1, conv_cache_std=1.0)
    s16 = inp["state_in"].to(torch.bfloat16)
    o_a, st_a, _ = _fused(dict(inp, state_in=s16))
    o_b, st_b, _ = _fused(dict(inp, state_in=s16.float()))
    assert torch.equal(o_a, o_b) and torch.equal(st_a, st_b.to(torch.bfloat16))
    slots = torch.tensor([5, 0, 3, 1], dtype=torch.int32, device=DEV)
    pool = seeded((6, H, 128, 128), 262)
    pool[slots.long()] = inp["state_in"]
    cpool = seeded((6, 3, 3 * H * 128), 263).to(torch.bfloat16)
    cpool[slots.long()] = inp["conv_state_in"]
    untouched = [r for r in range(6) if r not in slots.tolist()]
    keep_s, keep_c = pool[untouched].clone(), cpool[untouched].clone()
    o_p, _, _ = _fused(dict(inp, state_in=pool, conv_state_in=cpool), state_out=pool,
                       conv_state_out=cpool, state_slots=slots)
    o_w, st_w, cs_w = _fused(inp)
    assert torch.equal(o_p, o_w)
    assert torch.equal(pool[slots.long()], st_w) and torch.equal(cpool[slots.long()], cs_w)
    assert torch.equal(pool[untouched], keep_s) and torch.equal(cpool[untouched], keep_c)


def test_many_pairs_choose_the_fused_schedule():
    """With many (sequence, head) pairs (1024; the threshold is FUSED_MIN_PAIRS) the
    automatic choice is the fused schedule:
    the recommended workspace is 0 and the default call equals an explicit fused
    call bit for bit; an explicit two-pass call of the same input stays within
    the bar of it."""
    lengths = [40, 17, 64, 5] * 4
    H = 64
    inp = KI.make_prefill(H, lengths, seed=271, device=DEV, state_std=0.1)
    T = sum(lengths)
    assert kda.prefill_workspace_bytes(T, H, len(lengths)) == 0
    auto = _fused(inp, schedule="auto")
    fused = _fused(inp)
    assert torch.equal(auto[0], fused[0]) and torch.equal(auto[1], fused[1])
    two = _fused(inp, schedule="two_pass", workspace=True)
    heads = [0, 63]
    cu = inp["cu_seqlens"].cpu()
    from tests._gpu_common import head_conv_w
    ref = oracle.prefill(inp["q"][:, heads], inp["k"][:, heads], inp["v"][:, heads],
                         inp["gate"][:, heads], inp["beta"][:, heads],
                         head_conv_w(inp["conv_w"], H, heads), cu,
                         state_in=inp["state_in"][:, heads])
    for name, (o, st, _) in (("fused", fused), ("two-pass", two)):
        assert_bf16_close(o[:, heads], ref["o"], cu, len(heads), st[:, heads], ref["state"], name)


def test_more_sequences_than_the_length_order_ranks():
    """The fused and pass-B workgroups take sequences longest first when a call has
    at most 256 of them, and in index order beyond; 300 ragged sequences (empty
    ones among them) at 4 heads (1200 pairs: the fused schedule by default) take
    the index order, and match the oracle on both schedules; 200 of them take the
    length order and match as well."""
    H = 4
    for count, seed in ((300, 281), (200, 282)):
        lengths = [(7 * i + 3) % 41 for i in range(count)]
        inp = KI.make_prefill(H, lengths, seed=seed, device=DEV, state_std=0.1, conv_cache_std=1.0)
        ref = _oracle(inp)
        cu = inp["cu_seqlens"].cpu()
        if count * H >= kda.FUSED_MIN_PAIRS:
            assert kda.prefill_workspace_bytes(sum(lengths), H, count) == 0
        for sched in ("fused", "two_pass"):
            kw = {"workspace": True} if sched == "two_pass" else {}
            o, st, cs = _fused(inp, schedule=sched, **kw)
            assert_bf16_close(o, ref["o"], cu, H, st, ref["state"], "%d sequences, %s" % (count, sched))
            np.testing.assert_array_equal(to_np(cs), ref["conv_state"])


def test_ninety_six_heads_on_every_schedule_and_decode():
    """A head count above 64 and not a power of two (96: token rows of 48 KiB per
    tensor, conv channels 3 x 96 x 128) through the three prefill schedules and one
    decode step, against the oracle."""
    H, lengths = 96, [5, 40, 130]
    inp = KI.make_prefill(H, lengths, seed=291, device=DEV, state_std=0.1, conv_cache_std=1.0)
    ref = _oracle(inp)
    cu = inp["cu_seqlens"].cpu()
    for sched, kw in (("fused", {}), ("two_pass", {"workspace": True}), ("one_pass", {"workspace": None})):
        o, st, cs = _fused(inp, schedule=sched, **kw)
        assert_bf16_close(o, ref["o"], cu, H, st, ref["state"], "96 heads, " + sched)
        np.testing.assert_array_equal(to_np(cs), ref["conv_state"])
    d = KI.make_decode(5, H, seed=292, device=DEV)
    refd = oracle.decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"], d["conv_state"], d["state"])
    od = kda.kda_decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"], d["conv_state"], d["state"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(d["conv_state"]), refd["conv_state"])
    e = np.linalg.norm((to_np(od) - refd["o"]).reshape(-1, 128), axis=1) / \
        np.linalg.norm(refd["o"].reshape(-1, 128), axis=1)
    assert e.max() <= BF16_REL
    assert state_rel_errors(d["state"], refd["state"]).max() <= BF16_REL


def test_hand_over_waits_give_up_instead_of_hanging():
    """With the wait bound forced down to one poll from the host, the fused kernel's
    hand-over waits give up at once and mark their workgroup, whose waves then wait
    no more: the call ends (its results are not checked: a wave that gives up uses
    a ring slot before its hand-over).  With the default bound restored the same
    call equals its earlier result bit for bit."""
    lengths = [40, 17, 64, 5] * 4
    H = 64  # 1024 pairs: the fused schedule
    inp = KI.make_prefill(H, lengths, seed=301, device=DEV, state_std=0.1)
    ref = _fused(inp)
    prev = kda.set_spin_limit(1)
    try:
        o, st, cs = _fused(inp)  # must return
        assert o.shape == ref[0].shape
    finally:
        assert kda.set_spin_limit(0) == 1
    assert prev == kda.set_spin_limit(0)  # 0 restored the default
    again = _fused(inp)
    assert torch.equal(again[0], ref[0]) and torch.equal(again[1], ref[1]) and torch.equal(again[2], ref[2])


def test_automatic_choice_weighs_the_longest_sequence():
    """512 pairs: with one sequence much longer than the mean load per compute unit
    the automatic choice (host lengths given) is the two-pass schedule, bit for bit;
    with balanced lengths it is the fused schedule, bit for bit."""
    H = 64
    for lengths, want in (([2048] + [64] * 7, "two_pass"), ([256] * 8, "fused")):
        inp = KI.make_prefill(H, lengths, seed=311, device=DEV, state_std=0.1)
        cu_h = inp["cu_seqlens"].cpu()
        auto = _fused(inp, schedule="auto", cu_seqlens_host=cu_h, workspace=True)
        kw = {"workspace": True} if want == "two_pass" else {}
        ref = _fused(inp, schedule=want, cu_seqlens_host=cu_h, **kw)
        for a_, b_ in zip(auto, ref):
            assert torch.equal(a_, b_), want
