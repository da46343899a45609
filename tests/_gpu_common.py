"""Shared helpers for the GPU parity tests: tolerance checks against the oracle
and head/sequence sampling of large workloads."""
import numpy as np
import torch

# bf16 inputs: relative L2 error per (sequence, head) slice, max over slices
BF16_REL = 2e-2
# fp32 inputs: max absolute error
F32_ABS = 1e-4


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(t) else t


def slice_rel_errors(x, ref, cu, H):
    """Relative L2 error of o ([T, H, d]) per (sequence, head) slice."""
    x, ref = to_np(x), to_np(ref)
    cu = [int(c) for c in cu]
    errs = []
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        for h in range(H):
            d = np.linalg.norm(x[a:b, h] - ref[a:b, h])
            r = np.linalg.norm(ref[a:b, h])
            errs.append(d / max(r, 1e-30))
    return np.array(errs)


def state_rel_errors(x, ref):
    """Relative L2 error of states ([N, H, dk, dv]) per (sequence, head)."""
    x, ref = to_np(x), to_np(ref)
    N, H = ref.shape[:2]
    d = np.linalg.norm((x - ref).reshape(N * H, -1), axis=1)
    r = np.linalg.norm(ref.reshape(N * H, -1), axis=1)
    return d / np.maximum(r, 1e-30)


def assert_bf16_close(o, ref_o, cu, H, st=None, ref_st=None, what=""):
    e = slice_rel_errors(o, ref_o, cu, H)
    assert e.size == 0 or e.max() <= BF16_REL, "%s o rel err %.3g" % (what, e.max())
    if st is not None:
        es = state_rel_errors(st, ref_st)
        assert es.max() <= BF16_REL, "%s state rel err %.3g" % (what, es.max())


def assert_f32_close(x, ref, what=""):
    d = np.abs(to_np(x) - to_np(ref)).max() if np.size(ref) else 0.0
    assert d <= F32_ABS, "%s max abs err %.3g" % (what, d)


def head_conv_w(conv_w, H, heads, d=128):
    """Rows of a [3*H*d, 4] conv weight belonging to the given heads (q, k, v order)."""
    rows = []
    for part in range(3):
        for h in heads:
            base = part * H * d + h * d
            rows.append(conv_w[base:base + d])
    return torch.cat(rows, 0)


def head_conv_state(cs, H, heads, d=128):
    """Columns of a [N, 3, 3*H*d] conv state belonging to the given heads."""
    cols = []
    for part in range(3):
        for h in heads:
            base = part * H * d + h * d
            cols.append(cs[:, :, base:base + d])
    return torch.cat(cols, 2)


def seeded(shape, seed, kind="randn", device="cuda:0"):
    """A seeded draw on the host, moved to the device (test inputs are reproducible)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(shape, generator=g) if kind == "randn" else torch.rand(shape, generator=g)
    return x.to(device)
