"""Shared helpers for the GPU parity tests: tolerance checks against the oracle
and head/sequence selection of large workloads.

The bf16 bar (relative error 2e-2) is applied at two granularities:
  * per (sequence, head) slice of o and per (sequence, head) final state;
  * per block of 16 tokens of o inside each (sequence, head) slice, counted from
    the sequence start; a sequence's partial last block (1..15 tokens) joins the
    full block before it (a sequence shorter than 16 tokens is one block), so
    every block holds 16..31 tokens unless the whole sequence is shorter.  A
    relative L2 error over one to a few tokens measures single tokens whose
    output nearly cancels (|S^T q| much smaller than |S| |q|), where bf16 matrix
    operands err by more than 2e-2 of that small output on either schedule.
    The block's reference norm is floored at a tenth of the slice's
    root-mean-square block norm (a block whose true output is tiny is judged
    against the typical block of its slice, not against its own near-zero norm).
A single wrong 16-token block, or a few wrong tokens, therefore fails even in a
65,536-token slice, where they would move the slice norm by far less than 2e-2."""
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


BLOCK = 16          # tokens per block of the local bar
BLOCK_FLOOR = 0.1   # block reference norm floor, as a fraction of the slice RMS block norm


def block_rel_errors(x, ref, cu, H, block=BLOCK, floor=BLOCK_FLOOR):
    """Relative L2 error of o ([T, H, d]) per `block`-token block of every (sequence,
    head) slice (blocks counted from each sequence start; a partial last block joins
    the block before it).

    Returns (errors [num_blocks, H], block_starts [num_blocks]); the denominator of a
    block is max(|ref_block|, floor * slice RMS block norm)."""
    x, ref = to_np(x), to_np(ref)
    cu = [int(c) for c in cu]
    T = ref.shape[0]
    if T == 0:
        return np.zeros((0, H)), np.zeros(0, np.int64)
    # per token row: squared error and squared reference, [T, H]
    e2 = np.einsum("thd,thd->th", x - ref, x - ref)
    r2 = np.einsum("thd,thd->th", ref, ref)
    starts, seq_of = [], []
    for n in range(len(cu) - 1):
        L = cu[n + 1] - cu[n]
        for j in range(max(1, L // block) if L > 0 else 0):
            starts.append(cu[n] + block * j)
            seq_of.append(n)
    starts = np.asarray(starts, np.int64)
    be = np.add.reduceat(e2, starts, axis=0)
    br = np.add.reduceat(r2, starts, axis=0)
    seq_of = np.asarray(seq_of)
    den = np.sqrt(br)
    for n in range(len(cu) - 1):
        sel = seq_of == n
        if not sel.any():
            continue
        rms = np.sqrt(br[sel].mean(axis=0))  # per head
        den[sel] = np.maximum(den[sel], floor * rms[None, :])
    return np.sqrt(be) / np.maximum(den, 1e-30), starts


def assert_bf16_close(o, ref_o, cu, H, st=None, ref_st=None, what="", blocks=True):
    e = slice_rel_errors(o, ref_o, cu, H)
    assert e.size == 0 or e.max() <= BF16_REL, "%s o rel err %.3g" % (what, e.max())
    if blocks:
        eb, starts = block_rel_errors(o, ref_o, cu, H)
        if eb.size:
            i, h = np.unravel_index(int(np.argmax(eb)), eb.shape)
            assert eb.max() <= BF16_REL, "%s o rel err %.3g in the block at token %d, " \
                "head %d" % (what, eb.max(), int(starts[i]), int(h))
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
