"""GPU parity of the gate and beta in-projections (kda_gate_beta_proj) against
the fp64 oracle, and the fused path into the mixer.  Bar: bf16 relative L2 per
head (over tokens and channels) <= 2e-2 for the gate and for beta."""
import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
import gated_delta_rule_short_amd as kda
from tests._gpu_common import BF16_REL, slice_rel_errors, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_library()


def _per_head_rel(x, ref):
    """Relative L2 per head: x, ref [T, H, ...]."""
    x, ref = to_np(x), np.asarray(ref, np.float64)
    H = ref.shape[1]
    d = np.linalg.norm((x - ref).reshape(-1, H, int(np.prod(ref.shape[2:]) or 1)).transpose(1, 0, 2)
                       .reshape(H, -1), axis=1)
    r = np.linalg.norm(ref.reshape(-1, H, int(np.prod(ref.shape[2:]) or 1)).transpose(1, 0, 2)
                       .reshape(H, -1), axis=1)
    return d / np.maximum(r, 1e-30)


@pytest.mark.parametrize("T,hidden,H", [(1, 256, 64), (100, 512, 64), (333, 1024, 128),
                                        (70, 768, 128), (129, 4096, 64)])
@pytest.mark.parametrize("log", [False, True])
def test_gate_beta_proj_matches_oracle(T, hidden, H, log):
    d = KI.make_gate_proj(T, hidden=hidden, H=H, seed=110 + T, device=DEV)
    gate, beta = kda.kda_gate_beta_proj(d["x"], d["w_a"], d["w_b"], d["w_beta"], log=log)
    torch.cuda.synchronize()
    ref = oracle.gate_beta_proj(d["x"].cpu(), d["w_a"].cpu(), d["w_b"].cpu(), d["w_beta"].cpu(), H,
                                log=log)
    assert _per_head_rel(gate, ref["gate"]).max() <= BF16_REL
    assert _per_head_rel(beta[:, :, None], ref["beta"][:, :, None]).max() <= BF16_REL
    if log:  # the fused activation keeps the log-decay inside (lb, 0)
        assert float(gate.float().max()) <= 0.0 and float(gate.float().min()) >= -5.0


def test_gate_beta_proj_full_size():
    """The model's shape: 4096 tokens x hidden 4096 -> 64 heads x 128 gate channels."""
    d = KI.make_gate_proj(4096, seed=6, device=DEV)
    gate, beta = kda.kda_gate_beta_proj(d["x"], d["w_a"], d["w_b"], d["w_beta"], log=True)
    torch.cuda.synchronize()
    ref = oracle.gate_beta_proj(d["x"].cpu(), d["w_a"].cpu(), d["w_b"].cpu(), d["w_beta"].cpu(), 64,
                                log=True)
    assert _per_head_rel(gate, ref["gate"]).max() <= BF16_REL
    assert _per_head_rel(beta[:, :, None], ref["beta"][:, :, None]).max() <= BF16_REL


def test_gate_beta_proj_reuses_workspace_and_is_deterministic():
    d = KI.make_gate_proj(200, hidden=512, H=64, seed=120, device=DEV)
    ws = torch.empty(kda.gate_beta_workspace_bytes(200, 64), dtype=torch.uint8, device=DEV)
    g1, b1 = kda.kda_gate_beta_proj(d["x"], d["w_a"], d["w_b"], d["w_beta"], workspace=ws)
    g2, b2 = kda.kda_gate_beta_proj(d["x"], d["w_a"], d["w_b"], d["w_beta"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2) and torch.equal(b1, b2)


def test_projection_feeds_the_mixer():
    """x -> (gate as log-decay, beta) -> kda_prefill with KDA_F_GATE_IS_LOG, against the
    oracle chain (fp64 projection, then the oracle recurrence on its outputs)."""
    H, L = 64, [40, 90]
    T = sum(L)
    d = KI.make_gate_proj(T, hidden=512, H=H, seed=121, device=DEV)
    mix = KI.make_prefill(H, L, seed=122, device=DEV)
    gate, beta = kda.kda_gate_beta_proj(d["x"], d["w_a"], d["w_b"], d["w_beta"], log=True)
    o, _, _ = kda.kda_prefill(mix["q"], mix["k"], mix["v"], gate, beta, mix["conv_w"],
                              cu_seqlens=mix["cu_seqlens"], flags=kda.KDA_F_GATE_IS_LOG,
                              workspace=True)
    torch.cuda.synchronize()
    ref_p = oracle.gate_beta_proj(d["x"].cpu(), d["w_a"].cpu(), d["w_b"].cpu(), d["w_beta"].cpu(),
                                  H, log=True)
    ref = oracle.prefill(mix["q"], mix["k"], mix["v"], ref_p["gate"], ref_p["beta"], mix["conv_w"],
                         mix["cu_seqlens"], flags=oracle.GATE_IS_LOG)
    assert slice_rel_errors(o, ref["o"], mix["cu_seqlens"].cpu().tolist(), H).max() <= BF16_REL
