"""GPU tests of the state pool: slot-mapped prefill, decode, multi-token decode and
commit, and pool-row copies (prefix snapshot and fork).

A slot-mapped call must equal the same call on the gathered rows bit for bit and
leave every other pool row untouched; a forked prefix continued by decode must
match the oracle over prefix + continuation; a slot outside the pool skips its
sequence."""
import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import BF16_REL, seeded, slice_rel_errors, state_rel_errors, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _pool(rows, H, dtype, seed, sdt=torch.float32):
    """A state pool [rows, H, 128, 128] and a conv pool [rows, 3, 3*H*128]."""
    st = (0.1 * seeded((rows, H, 128, 128), seed)).to(sdt)
    cs = seeded((rows, 3, 3 * H * 128), seed + 1).to(dtype)
    return st, cs


def _untouched(pool, before, used):
    keep = [r for r in range(pool.shape[0]) if r not in used]
    return torch.equal(pool[keep], before[keep])


@pytest.mark.parametrize("sdt", [torch.float32, torch.bfloat16])
def test_decode_with_slots_equals_gathered_rows(sdt):
    N, H, P = 3, 3, 7
    d = KI.make_decode(N, H, seed=91, device=DEV)
    st, cs = _pool(P, H, torch.bfloat16, 92, sdt)
    slots = [5, 0, 3]
    sl = torch.tensor(slots, dtype=torch.int32, device=DEV)
    st0, cs0 = st.clone(), cs.clone()
    g_st, g_cs = st[slots].clone(), cs[slots].clone()
    args = (d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"])
    o_ref = kda.kda_decode(*args, g_cs, g_st)
    o = kda.kda_decode(*args, cs, st, state_slots=sl)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(st[slots], g_st) and torch.equal(cs[slots], g_cs)
    assert _untouched(st, st0, slots) and _untouched(cs, cs0, slots)


def test_multi_and_commit_with_slots():
    N, H, T, P = 4, 2, 6, 9
    d = KI.make_spec_decode(N, T, H, seed=93, device=DEV)
    st, cs = _pool(P, H, torch.bfloat16, 94)
    slots = [8, 2, 6, 1]
    sl = torch.tensor(slots, dtype=torch.int32, device=DEV)
    st0, cs0 = st.clone(), cs.clone()
    g_st, g_cs = st[slots].clone(), cs[slots].clone()
    args = (d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"])
    acc = torch.tensor([1, 6, 0, 3], dtype=torch.int32, device=DEV)
    o_ref, u_ref = kda.kda_decode_multi(*args, g_cs, g_st)
    kda.kda_decode_commit(u_ref, acc, g_cs, g_st)
    o, u = kda.kda_decode_multi(*args, cs, st, state_slots=sl)
    kda.kda_decode_commit(u, acc, cs, st, state_slots=sl)
    # the fused form on a second copy of the pool: step two commits step one
    st2, cs2 = st0.clone(), cs0.clone()
    _, u1 = kda.kda_decode_multi(*args, cs2, st2, state_slots=sl)
    o2, _ = kda.kda_decode_multi(*args, cs2, st2, state_slots=sl, pending_updates=u1,
                                 pending_accepted=acc)
    o2_ref, _ = kda.kda_decode_multi(*args, g_cs, g_st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(u, u_ref)
    assert torch.equal(st[slots], g_st) and torch.equal(cs[slots], g_cs)
    assert _untouched(st, st0, slots) and _untouched(cs, cs0, slots)
    assert torch.equal(o2, o2_ref)
    assert torch.equal(st2, st) and torch.equal(cs2, cs)


@pytest.mark.parametrize("dtype,kw", [(torch.bfloat16, {"workspace": True}),
                                      (torch.bfloat16, {"chunk_size": 64}),
                                      (torch.float32, {"chunk_size": 16})])
def test_prefill_with_slots_in_place(dtype, kw):
    H, P = 2, 6
    inp = KI.make_prefill(H, [37, 0, 70], dtype=dtype, seed=95, device=DEV)
    st, cs = _pool(P, H, dtype, 96)
    slots = [4, 1, 2]
    sl = torch.tensor(slots, dtype=torch.int32, device=DEV)
    st0, cs0 = st.clone(), cs.clone()
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"])
    g_st, g_cs = st[slots].clone(), cs[slots].clone()
    o_ref, st_ref, cs_ref = kda.kda_prefill(*args, cu_seqlens=inp["cu_seqlens"], state_in=g_st,
                                            conv_state_in=g_cs, state_out=True,
                                            conv_state_out=True, **kw)
    o, _, _ = kda.kda_prefill(*args, cu_seqlens=inp["cu_seqlens"], state_in=st, state_out=st,
                              conv_state_in=cs, conv_state_out=cs, state_slots=sl, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(st[slots], st_ref) and torch.equal(cs[slots], cs_ref)
    assert _untouched(st, st0, slots) and _untouched(cs, cs0, slots)


def test_slot_outside_pool_skips_the_sequence():
    N, H, P = 3, 2, 4
    d = KI.make_decode(N, H, seed=97, device=DEV)
    st, cs = _pool(P, H, torch.bfloat16, 98)
    st0, cs0 = st.clone(), cs.clone()
    sl = torch.tensor([2, -1, P], dtype=torch.int32, device=DEV)
    o = torch.full_like(d["v"], 7.0)
    kda.kda_decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"], cs, st, o=o,
                   state_slots=sl)
    torch.cuda.synchronize()
    assert torch.all(o[1:] == 7.0) and not torch.all(o[0] == 7.0)
    assert _untouched(st, st0, [2]) and _untouched(cs, cs0, [2])


@pytest.mark.parametrize("sched", ["fused", "two_pass", "one_pass"])
def test_prefill_slot_outside_pool_skips_the_sequence(sched):
    """Prefill on every schedule: sequences with slots -1 and num_slots write no
    output, state or conv state; the valid one equals the same call with every slot
    valid, bit for bit."""
    H, P = 2, 4
    inp = KI.make_prefill(H, [20, 33, 17], seed=101, device=DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"])
    kw = {"workspace": True} if sched == "two_pass" else {}
    cu = [int(c) for c in inp["cu_seqlens"].cpu()]

    def run(slots, st, cs):
        o = torch.full_like(inp["v"], 7.0)
        kda.kda_prefill(*args, cu_seqlens=inp["cu_seqlens"], state_in=st, state_out=st, conv_state_in=cs,
                        conv_state_out=cs, state_slots=torch.tensor(slots, dtype=torch.int32, device=DEV),
                        o=o, schedule=sched, **kw)
        torch.cuda.synchronize()
        return o

    st, cs = _pool(P, H, torch.bfloat16, 102)
    st0, cs0 = st.clone(), cs.clone()
    o = run([2, -1, P], st, cs)
    assert torch.all(o[cu[1]:] == 7.0) and not torch.all(o[:cu[1]] == 7.0)
    assert _untouched(st, st0, [2]) and _untouched(cs, cs0, [2])
    st_v, cs_v = st0.clone(), cs0.clone()
    o_v = run([2, 0, 1], st_v, cs_v)
    assert torch.equal(o[:cu[1]], o_v[:cu[1]])
    assert torch.equal(st[2], st_v[2]) and torch.equal(cs[2], cs_v[2])


@pytest.mark.parametrize("sdt", [torch.float32, torch.bfloat16])
def test_state_copy(sdt):
    H, P = 3, 8
    st, cs = _pool(P, H, torch.bfloat16, 99, sdt)
    st0, cs0 = st.clone(), cs.clone()
    src = torch.tensor([1, 4, 7, 5], dtype=torch.int32, device=DEV)
    dst = torch.tensor([6, 2, -1, 5], dtype=torch.int32, device=DEV)  # -1: skipped; 5 -> 5: no-op
    kda.kda_state_copy(st, src, dst, conv_pool=cs)
    torch.cuda.synchronize()
    assert torch.equal(st[6], st0[1]) and torch.equal(st[2], st0[4])
    assert torch.equal(cs[6], cs0[1]) and torch.equal(cs[2], cs0[4])
    assert _untouched(st, st0, [6, 2]) and _untouched(cs, cs0, [6, 2])
    # into a second pool, state only
    st_b = torch.zeros_like(st)
    kda.kda_state_copy(st, src[:2], dst[:2], dst_state_pool=st_b)
    torch.cuda.synchronize()
    assert torch.equal(st_b[6], st[1]) and torch.equal(st_b[2], st[4])
    assert int((st_b[[0, 1, 3, 4, 5, 7]] != 0).sum()) == 0


def test_prefix_fork_then_decode_matches_oracle():
    """Prefill a shared prefix into slot 0, fork it to slots 3 and 5, and continue each
    with its own tokens by decode; each branch equals the oracle over prefix +
    continuation."""
    H, Lp, Td, P = 2, 45, 4, 6
    pre = KI.make_prefill(H, [Lp], seed=100, device=DEV, state_std=0.1, conv_cache_std=1.0)
    cont = KI.make_prefill(H, [Td, Td], seed=101, device=DEV)
    cont["conv_w"] = pre["conv_w"]
    st = torch.zeros((P, H, 128, 128), device=DEV)
    cs = torch.zeros((P, 3, 3 * H * 128), dtype=torch.bfloat16, device=DEV)
    st[0] = pre["state_in"][0]
    cs[0] = pre["conv_state_in"][0]
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.kda_prefill(pre["q"], pre["k"], pre["v"], pre["gate"], pre["beta"], pre["conv_w"],
                    cu_seqlens=pre["cu_seqlens"], state_in=st, state_out=st, conv_state_in=cs,
                    conv_state_out=cs, state_slots=zero, workspace=True)
    kda.kda_state_copy(st, torch.tensor([0, 0], dtype=torch.int32, device=DEV),
                       torch.tensor([3, 5], dtype=torch.int32, device=DEV), conv_pool=cs)
    sl = torch.tensor([3, 5], dtype=torch.int32, device=DEV)
    view = lambda x: x.view(2, Td, *x.shape[1:])
    outs = []
    for t in range(Td):
        outs.append(kda.kda_decode(*(view(cont[n])[:, t].contiguous()
                                     for n in ("q", "k", "v", "gate", "beta")),
                                   cont["conv_w"], cs, st, state_slots=sl))
    torch.cuda.synchronize()
    for b in range(2):
        cat = lambda n: torch.cat([pre[n].cpu(), view(cont[n])[b].cpu()], 0)
        ref = oracle.prefill(cat("q"), cat("k"), cat("v"), cat("gate"), cat("beta"),
                             pre["conv_w"], np.array([0, Lp + Td], np.int32),
                             state_in=pre["state_in"].cpu(),
                             conv_state_in=pre["conv_state_in"].cpu())
        o_b = torch.stack([outs[t][b] for t in range(Td)])
        assert slice_rel_errors(o_b, ref["o"][Lp:], [0, Td], H).max() <= BF16_REL
        assert state_rel_errors(st[3 + 2 * b:4 + 2 * b], ref["state"]).max() <= BF16_REL
        np.testing.assert_array_equal(to_np(cs[3 + 2 * b:4 + 2 * b]), ref["conv_state"])
