"""Full-size GPU parity: every (sequence, head) pair of the three prefill workloads
(1 x 4096 tokens; 1 x 65,536 tokens with decays near the bound; 16 packed
sequences of 512..16,384 tokens with initial states) and every sequence of the
256-sequence decode step, on every prefill schedule (the benchmark times the
automatic choice: two passes for the single sequences, fused for the 16), against
the fp64 oracle.

o is checked per (sequence, head) slice and per 16-token block of each slice
(relative L2 <= 2e-2, see tests/_gpu_common.py); the final state per (sequence,
head); the final conv state bit for bit.  The oracle runs over groups of 16
heads so that its float64 copies stay a few GB."""
import sys
import time

import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import (BF16_REL, assert_bf16_close, head_conv_state, head_conv_w,
                               state_rel_errors, to_np)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GROUP = 16  # heads per oracle call


def _progress(msg):
    # straight to the terminal (pytest captures sys.stderr): a long test reports each step
    sys.__stderr__.write("[fullsize %.1fs] %s\n" % (time.perf_counter(), msg))
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _schedules():
    # the three schedules: two passes (the default for few pairs), fused (the
    # default from FUSED_MIN_PAIRS pairs on) and one pass with 64-token chunks
    return {"two_pass": {"schedule": "two_pass"}, "fused": {"schedule": "fused"},
            "one_pass_chunk64": {"chunk_size": 64, "workspace": None, "schedule": "one_pass"}}


def _run_gpu(inp, **kw):
    o, st, cs = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                inp["conv_w"], cu_seqlens=inp["cu_seqlens"],
                                state_in=inp.get("state_in"),
                                conv_state_in=inp.get("conv_state_in"), state_out=True,
                                conv_state_out=True, **kw)
    torch.cuda.synchronize()
    return o, st, cs


def _check_all_heads(inp, results):
    H = inp["H"]
    cu = inp["cu_seqlens"].cpu()
    worst = {name: [0.0, 0.0] for name in results}
    for h0 in range(0, H, GROUP):
        heads = list(range(h0, min(H, h0 + GROUP)))
        ref = oracle.prefill(inp["q"][:, heads], inp["k"][:, heads], inp["v"][:, heads],
                             inp["gate"][:, heads], inp["beta"][:, heads],
                             head_conv_w(inp["conv_w"], H, heads), cu,
                             state_in=None if inp.get("state_in") is None
                             else inp["state_in"][:, heads],
                             conv_state_in=None if inp.get("conv_state_in") is None
                             else head_conv_state(inp["conv_state_in"], H, heads))
        for name, (o, st, cs) in results.items():
            what = "%s heads %d..%d" % (name, heads[0], heads[-1])
            assert torch.isfinite(o[:, heads]).all() and torch.isfinite(st[:, heads]).all(), what
            assert_bf16_close(o[:, heads], ref["o"], cu, len(heads), st[:, heads], ref["state"],
                              what)
            np.testing.assert_array_equal(to_np(head_conv_state(cs, H, heads)),
                                          ref["conv_state"], err_msg=what)
            worst[name][1] = max(worst[name][1], float(state_rel_errors(st[:, heads],
                                                                         ref["state"]).max()))
        _progress("heads %d..%d checked" % (heads[0], heads[-1]))
        del ref
    return worst


@pytest.mark.timeout(900)
@pytest.mark.parametrize("workload", [1, 3, 4])
def test_prefill_full_size_every_head(workload):
    inp = KI.workload_inputs(workload, device=DEV)
    _progress("workload %d: %d tokens, %d sequences" % (workload, inp["q"].shape[0],
                                                         len(inp["lengths"])))
    results = {name: _run_gpu(inp, **kw) for name, kw in _schedules().items()}
    _progress("workload %d: every schedule ran" % workload)
    worst = _check_all_heads(inp, results)
    print("workload %d: worst final-state rel err %s" % (workload, worst))


@pytest.mark.timeout(600)
def test_decode_full_size_every_sequence():
    """The 256-sequence x 64-head decode step as timed, every sequence checked."""
    d = KI.workload_inputs(2, device=DEV)
    st0 = d["state"].clone()
    cs0 = d["conv_state"].clone()
    o = kda.kda_decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["conv_w"], d["conv_state"],
                       d["state"])
    torch.cuda.synchronize()
    N = o.shape[0]
    for n0 in range(0, N, 32):
        sl = slice(n0, n0 + 32)
        ref = oracle.decode(d["q"][sl], d["k"][sl], d["v"][sl], d["gate"][sl], d["beta"][sl],
                            d["conv_w"], cs0[sl], st0[sl])
        # one token per (sequence, head): the relative error of each output row
        e = np.linalg.norm((to_np(o[sl]) - ref["o"]).reshape(-1, 128), axis=1) / \
            np.linalg.norm(ref["o"].reshape(-1, 128), axis=1)
        assert e.max() <= BF16_REL, (n0, e.max())
        assert state_rel_errors(d["state"][sl], ref["state"]).max() <= BF16_REL, n0
        np.testing.assert_array_equal(to_np(d["conv_state"][sl]), ref["conv_state"])
