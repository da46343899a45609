"""Two-pass prefill in windows: a workspace smaller than the whole call runs the
call in windows of sub-chunks, every sequence advancing together, with the fp32
state carried between windows.  The windowed result must equal the whole call's
bit for bit (same arithmetic, the state only waits in fp32 memory), on both
pass-B geometries, with bf16 state storage and with a state pool; and a prompt of
260,408 tokens (the longest prompt of the serving battery in "GLM-5.3-Flash
Internals") runs within the capped workspace and matches the oracle on sampled
heads."""
import sys
import time

import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import assert_bf16_close, head_conv_w, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CARRY = 128 * 128 * 4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _window_ws(N, H, jw):
    """A workspace of exactly jw sub-chunks per sequence and head plus the carry."""
    rec = kda.prefill_workspace_bytes(16, 1, 1, which="full") // 2  # bytes of one record
    return torch.empty(N * H * (jw * rec + CARRY), dtype=torch.uint8, device=DEV)


def _run(inp, ws, host_cu=True, **kw):
    o, st, cs = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                inp["conv_w"], cu_seqlens=inp["cu_seqlens"],
                                cu_seqlens_host=inp["cu_seqlens"].cpu() if host_cu else None,
                                state_in=inp.get("state_in"), conv_state_in=inp.get("conv_state_in"),
                                state_out=True, conv_state_out=True, workspace=ws, **kw)
    torch.cuda.synchronize()
    return o, st, cs


LENGTHS = [1, 0, 17, 64, 130, 200, 33]


@pytest.mark.parametrize("jw", [1, 2, 5])
@pytest.mark.parametrize("dv_tile", [16, 32, 128])
@pytest.mark.parametrize("host_cu", [True, False])
def test_windows_equal_whole_call_bitwise(jw, dv_tile, host_cu):
    H = 3
    inp = KI.make_prefill(H, LENGTHS, seed=181, device=DEV, state_std=0.1, conv_cache_std=1.0)
    whole = _run(inp, True, dv_tile=dv_tile)
    win = _run(inp, _window_ws(len(LENGTHS), H, jw), host_cu=host_cu, dv_tile=dv_tile)
    for a, b, nm in zip(whole, win, ("o", "state", "conv state")):
        assert torch.equal(a, b), nm
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"],
                         inp["cu_seqlens"], state_in=inp["state_in"],
                         conv_state_in=inp["conv_state_in"])
    assert_bf16_close(win[0], ref["o"], inp["cu_seqlens"].cpu(), H, win[1], ref["state"], "windows")


def test_windows_bf16_state_and_pool_bitwise():
    """bf16 state storage rounds once at the end of the call, not per window (the
    carry is fp32); pool slots map each sequence's state rows in every window."""
    H, N = 2, len(LENGTHS)
    inp = KI.make_prefill(H, LENGTHS, seed=182, device=DEV, state_std=0.1, conv_cache_std=1.0)
    s16 = inp["state_in"].to(torch.bfloat16)
    args = (inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["conv_w"])
    common = dict(cu_seqlens=inp["cu_seqlens"], cu_seqlens_host=inp["cu_seqlens"].cpu(),
                  conv_state_in=inp["conv_state_in"], state_in=s16, state_out=True)
    o_a, st_a, _ = kda.kda_prefill(*args, workspace=True, **common)
    o_b, st_b, _ = kda.kda_prefill(*args, workspace=_window_ws(N, H, 2), **common)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(st_a, st_b)
    # a pool of 11 rows, sequence n in row slots[n]
    slots = torch.tensor([9, 0, 4, 7, 2, 10, 5], dtype=torch.int32, device=DEV)
    pool = torch.zeros((11, H, 128, 128), device=DEV)
    pool[slots.long()] = inp["state_in"]
    cpool = torch.zeros((11, 3, 3 * H * 128), dtype=torch.bfloat16, device=DEV)
    cpool[slots.long()] = inp["conv_state_in"]
    o_p, _, _ = kda.kda_prefill(*args, cu_seqlens=inp["cu_seqlens"],
                                cu_seqlens_host=inp["cu_seqlens"].cpu(), state_in=pool,
                                state_out=pool, conv_state_in=cpool, conv_state_out=cpool,
                                state_slots=slots, workspace=_window_ws(N, H, 3))
    o_w, st_w, cs_w = _run(inp, True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_w)
    assert torch.equal(pool[slots.long()], st_w) and torch.equal(cpool[slots.long()], cs_w)


def _progress(msg):
    sys.__stderr__.write("[windows %.1fs] %s\n" % (time.perf_counter(), msg))
    sys.__stderr__.flush()


@pytest.mark.timeout(600)
def test_prompt_of_260408_tokens_within_the_cap():
    """One sequence of 260,408 tokens, 64 heads (the whole call would need 14.4 GB of
    workspace): the recommended workspace stays within the cap, the call runs in
    windows, and sampled heads match the oracle per 16-token block."""
    T, H = 260408, 64
    inp = KI.make_prefill(H, [T], seed=260, device=DEV, state_std=0.1)
    cu_h = inp["cu_seqlens"].cpu()
    full = kda.prefill_workspace_bytes(T, H, 1, which="full")
    rec = kda.prefill_workspace_bytes(T, H, 1, cu_seqlens_host=cu_h)
    assert full > kda.PREFILL_WORKSPACE_CAP >= rec
    _progress("inputs ready, workspace %.2f GB (whole call %.2f GB)" % (rec / 1e9, full / 1e9))
    o, st, _ = _run(inp, torch.empty(rec, dtype=torch.uint8, device=DEV))
    assert torch.isfinite(o).all() and torch.isfinite(st).all()
    _progress("prefill ran")
    heads = [0, 37]
    ref = oracle.prefill(inp["q"][:, heads], inp["k"][:, heads], inp["v"][:, heads],
                         inp["gate"][:, heads], inp["beta"][:, heads],
                         head_conv_w(inp["conv_w"], H, heads), cu_h,
                         state_in=inp["state_in"][:, heads])
    _progress("oracle ran")
    assert_bf16_close(o[:, heads], ref["o"], cu_h, len(heads), st[:, heads], ref["state"],
                      "260,408 tokens")
