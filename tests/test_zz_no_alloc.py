"""kda_prefill_noalloc (the prefill entry point that allocates nothing, for callers
that cannot: graph capture, tight serving loops) against kda_prefill, through the
C ABI: two calls in a row on one GPU's scratch, the second with a smaller input.

The first call (1 x 6144 tokens, 64 heads) needs more two-pass workspace than the
scratch holds, so it runs in windows; the second (three short sequences, 4 heads)
fits at once and leaves most of the first call's scratch contents in place.  Both
must equal kda_prefill with a whole-call workspace bit for bit (the same kernels;
windows carry the fp32 state exactly), and so stay within the oracle's bar.  A
one-pass call (fp32 inputs) through the same entry point needs no scratch."""
import ctypes

import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from gated_delta_rule_short_amd import kda as K
from tests._gpu_common import assert_bf16_close, assert_f32_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _both(inp, **kw):
    outs = []
    for fn in (kda.kda_prefill, kda.kda_prefill_noalloc):
        o = torch.full_like(inp["v"], float("nan"))
        N, H = len(inp["lengths"]), inp["H"]
        st = torch.full((N, H, 128, 128), float("nan"), device=DEV)
        cs = torch.empty((N, 3, 3 * H * 128), dtype=inp["q"].dtype, device=DEV)
        fn(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
           cu_seqlens=inp["cu_seqlens"], cu_seqlens_host=inp["cu_seqlens"].cpu(),
           state_in=inp.get("state_in"), conv_state_in=inp.get("conv_state_in"), o=o,
           state_out=st, conv_state_out=cs, **kw)
        torch.cuda.synchronize()
        outs.append((o, st, cs))
    return outs


def test_noalloc_equals_prefill_twice_second_smaller():
    big = KI.workload_inputs(1, device=DEV, T=6144)  # 1 x 6144 tokens, 64 heads: windows in the scratch
    assert kda.prefill_workspace_bytes(6144, 64, 1, which="full") > kda.PREFILL_SCRATCH_BYTES
    (o_a, st_a, cs_a), (o_b, st_b, cs_b) = _both(big)
    assert torch.equal(o_a, o_b) and torch.equal(st_a, st_b) and torch.equal(cs_a, cs_b)
    small = KI.make_prefill(4, [300, 17, 65], seed=191, device=DEV, state_std=0.1,
                            conv_cache_std=1.0)
    (o_a, st_a, cs_a), (o_b, st_b, cs_b) = _both(small)
    assert torch.equal(o_a, o_b) and torch.equal(st_a, st_b) and torch.equal(cs_a, cs_b)
    ref = oracle.prefill(small["q"], small["k"], small["v"], small["gate"], small["beta"],
                         small["conv_w"], small["cu_seqlens"], state_in=small["state_in"],
                         conv_state_in=small["conv_state_in"])
    assert_bf16_close(o_b, ref["o"], small["cu_seqlens"].cpu(), 4, st_b, ref["state"], "noalloc")
    np.testing.assert_array_equal(cs_b.float().cpu().numpy(), ref["conv_state"])


def test_noalloc_one_pass_inputs_need_no_scratch():
    inp = KI.make_prefill(2, [40, 77], dtype=torch.float32, seed=192, device=DEV, state_std=0.1)
    (o_a, st_a, _), (o_b, st_b, _) = _both(inp, chunk_size=32)
    assert torch.equal(o_a, o_b) and torch.equal(st_a, st_b)
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                         inp["cu_seqlens"], state_in=inp["state_in"])
    assert_f32_close(o_b, ref["o"], "o")


def test_noalloc_rejects_a_workspace_and_calls_beyond_the_scratch():
    lib = kda.load_library()
    a = K.KdaPrefillArgs(num_seqs=1, num_heads=2, head_dim_k=128, head_dim_v=128,
                         total_tokens=64, dtype=kda.KDA_BF16, gate_lower_bound=-5.0)
    for f in ("q", "k", "v", "gate", "beta", "conv_weight", "o"):
        setattr(a, f, ctypes.c_void_p(0x100000))
    a.workspace, a.workspace_bytes = ctypes.c_void_p(0x200000), 1 << 20
    assert lib.kda_prefill_noalloc(ctypes.byref(a), None) == K.KDA_ERR_INVALID_ARG
    assert b"no workspace" in lib.kda_last_error()
    # an explicit two-pass call whose smallest workspace exceeds the scratch (the
    # automatic choice for these 262,144 pairs is the fused schedule, which needs none)
    b = K.KdaPrefillArgs(num_seqs=4096, num_heads=64, head_dim_k=128, head_dim_v=128,
                         total_tokens=4096 * 64, dtype=kda.KDA_BF16, gate_lower_bound=-5.0,
                         schedule=kda.SCHEDULES["two_pass"])
    assert lib.kda_prefill_workspace_min_size(ctypes.byref(b)) > kda.PREFILL_SCRATCH_BYTES
    assert lib.kda_prefill_noalloc(ctypes.byref(b), None) == K.KDA_ERR_INVALID_ARG
    assert b"scratch" in lib.kda_last_error()
