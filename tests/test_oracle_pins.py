"""Pins for the fp64 oracle, each against something other than the oracle itself:
a library routine, a closed form the mathematics fixes, brute-force unrolled
matrix products, or an exact invariant.  CPU only.

The mixer's definition followed by the oracle is the KDA passage of
"GLM-5.3-Flash im Detail" (section "Sequenz-Mixing: 34 KDA-Schichten mit
festem Zustand"): width-4 causal depthwise conv on q, k, v; channel-wise forget
gate with log-decay >= -5; scalar-beta delta-rule write; query read of the
updated state.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)
IDENT = np.array([0.0, 0.0, 0.0, 1.0])  # conv taps that pass the current token through


def _conv_lib(x, w, bias=None, hist=None, silu=False):
    """Reference conv via torch conv1d(groups=C) in fp64.  x: [L, C]; w: [C, 4];
    hist: [3, C] oldest first (or zeros)."""
    L, C = x.shape
    if hist is None:
        hist = np.zeros((3, C))
    if L == 0:
        return np.zeros((0, C))
    xp = torch.from_numpy(np.concatenate([hist, x], 0).T[None].copy())  # [1, C, L+3]
    wt = torch.from_numpy(w[:, None, :].copy())
    b = None if bias is None else torch.from_numpy(bias.copy())
    y = F.conv1d(xp, wt, b, groups=C)[0].T
    if silu:
        y = F.silu(y)
    return y.numpy()


# ---------------------------------------------------------------- short conv

@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_short_conv_matches_torch_conv1d(silu, with_state):
    C = 37
    lengths = [5, 1, 0, 2, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = cu[-1]
    x = RNG.standard_normal((T, C))
    w = RNG.standard_normal((C, 4))
    bias = RNG.standard_normal(C)
    cs = RNG.standard_normal((len(lengths), 3, C)) if with_state else None
    y, cso = oracle.short_conv(x, w, cu, bias=bias, conv_state_in=cs, silu=silu)
    for n, L in enumerate(lengths):
        s0 = cu[n]
        hist = cs[n] if with_state else np.zeros((3, C))
        ref = _conv_lib(x[s0:s0 + L], w, bias, hist, silu)
        np.testing.assert_allclose(y[s0:s0 + L], ref, rtol=1e-13, atol=1e-13)
        full = np.concatenate([hist, x[s0:s0 + L]], 0)
        np.testing.assert_array_equal(cso[n], full[-3:])


@pytest.mark.parametrize("tap", [0, 1, 2, 3])
def test_short_conv_one_hot_taps_shift_exactly(tap):
    C, T = 8, 11
    x = RNG.standard_normal((T, C))
    w = np.zeros((C, 4))
    w[:, tap] = 1.0
    y, _ = oracle.short_conv(x, w, np.array([0, T], np.int32))
    shift = 3 - tap
    expect = np.zeros_like(x)
    expect[shift:] = x[:T - shift]
    np.testing.assert_array_equal(y, expect)


# ------------------------------------------------------- helpers for prefill

def _ident_conv(H, dk, dv):
    return np.tile(IDENT, (2 * H * dk + H * dv, 1))


def _run(q, k, v, a, beta, lengths=None, conv_w=None, flags=0, **kw):
    T, H, dk = q.shape
    dv = v.shape[2]
    if lengths is None:
        lengths = [T]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if conv_w is None:
        conv_w = _ident_conv(H, dk, dv)
    return oracle.prefill(q, k, v, a, beta, conv_w, cu, flags=flags, **kw)


# --------------------------------------------------------- L2 and the gate

def test_l2_norm_closed_form():
    """One token, beta=1, no decay, q=k: o = scale * v * s/(s+eps), s = |k|^2,
    and the written state column is k_hat with |k_hat|^2 = s/(s+eps)."""
    H, dk, dv = 3, 16, 5
    for s_target in [1e-8, 1e-6, 0.3, 1.0, 77.0]:
        k = RNG.standard_normal((1, H, dk))
        k *= np.sqrt(s_target) / np.linalg.norm(k, axis=-1, keepdims=True)
        v = RNG.standard_normal((1, H, dv))
        out = _run(k, k, v, np.zeros((1, H, dk)), np.ones((1, H)), flags=oracle.GATE_IS_LOG,
                   scale=0.25)
        s = np.sum(k[0] ** 2, -1)
        np.testing.assert_allclose(out["o"][0], 0.25 * v[0] * (s / (s + 1e-6))[:, None],
                                   rtol=1e-12, atol=1e-300)
        col = out["state"][0, :, :, 0] / v[0, :, 0][:, None]
        np.testing.assert_allclose(np.sum(col ** 2, -1), s / (s + 1e-6), rtol=1e-12)
        off = _run(k, k, v, np.zeros((1, H, dk)), np.ones((1, H)),
                   flags=oracle.GATE_IS_LOG | oracle.NO_QK_L2NORM, scale=0.25)
        np.testing.assert_allclose(off["o"][0], 0.25 * v[0] * s[:, None], rtol=1e-12)


def test_gate_sigmoid_values_and_row_axis():
    """beta=0 single token: S1 = diag(exp(-5*sigmoid(a))) S0, decay on the dk rows.
    a=0 gives exactly exp(-2.5); a -> +inf gives exp(-5); a -> -inf gives 1."""
    H, dk, dv = 2, 8, 6
    a = RNG.standard_normal((1, H, dk)) * 3
    a[0, 0, :4] = [0.0, 60.0, -60.0, 1e4]
    S0 = RNG.standard_normal((1, H, dk, dv))
    z = np.zeros((1, H, dk))
    out = _run(z, z, np.zeros((1, H, dv)), a, np.zeros((1, H)), state_in=S0)
    alpha = np.exp(-5.0 * scipy.special.expit(a[0]))
    np.testing.assert_allclose(out["state"][0], alpha[:, :, None] * S0[0], rtol=1e-14)
    np.testing.assert_allclose(alpha[0, :3], [np.exp(-2.5), np.exp(-5.0), 1.0], rtol=1e-14)
    assert np.all(np.exp(-5.0) <= alpha) and np.all(alpha <= 1.0)
    # explicit log-gate with the clamp at the lower bound
    a2 = np.array([[[-7.0, -5.0, -1.0, 0.0, -4.99, -100.0, -0.1, -3.0]] * H]).reshape(1, H, dk)
    out2 = _run(z, z, np.zeros((1, H, dv)), a2, np.zeros((1, H)), state_in=S0,
                flags=oracle.GATE_IS_LOG)
    np.testing.assert_allclose(out2["state"][0], np.exp(np.maximum(a2[0], -5.0))[:, :, None] * S0[0],
                               rtol=1e-14)


# ------------------------------------------------ closed forms of the recurrence

def test_beta_zero_is_pure_gated_decay():
    """beta=0: no writes; o_t = scale S0^T (q_t * exp(sum_{s<=t} g_s)), S_L = diag(exp(sum g)) S0."""
    T, H, dk, dv = 23, 2, 16, 12
    q = RNG.standard_normal((T, H, dk))
    k = RNG.standard_normal((T, H, dk))
    v = RNG.standard_normal((T, H, dv))
    g = -5.0 * RNG.random((T, H, dk))
    S0 = RNG.standard_normal((1, H, dk, dv))
    out = _run(q, k, v, g, np.zeros((T, H)), state_in=S0, scale=0.7,
               flags=oracle.GATE_IS_LOG | oracle.NO_QK_L2NORM)
    cum = np.cumsum(g, 0)
    for t in range(T):
        ref = 0.7 * np.einsum("hi,hij->hj", q[t] * np.exp(cum[t]), S0[0])
        np.testing.assert_allclose(out["o"][t], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["state"][0], np.exp(cum[-1])[:, :, None] * S0[0], rtol=1e-12)


def test_one_hot_keys_reduce_to_gla():
    """Distinct one-hot keys and S0=0: the erase term vanishes and every written row only
    decays afterwards, so o_t = scale sum_{s<=t} q_t[pi_s] beta_s v_s prod_{s<u<=t} alpha_u[pi_s].
    The decay index pi_s is the dk channel of the key: this pins the gate's axis."""
    T, H, dk, dv = 40, 2, 64, 9
    pi = np.stack([RNG.permutation(dk)[:T] for _ in range(H)], 1)  # [T, H]
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            k[t, h, pi[t, h]] = 1.0
    q = RNG.standard_normal((T, H, dk))
    v = RNG.standard_normal((T, H, dv))
    g = -5.0 * RNG.random((T, H, dk))
    beta = RNG.random((T, H))
    out = _run(q, k, v, g, beta, scale=1.3, flags=oracle.GATE_IS_LOG | oracle.NO_QK_L2NORM)
    alpha = np.exp(g)
    for h in range(H):
        for t in range(T):
            ref = np.zeros(dv)
            for s in range(t + 1):
                c = pi[s, h]
                decay = np.prod(alpha[s + 1:t + 1, h, c])
                ref += q[t, h, c] * beta[s, h] * v[s, h] * decay
            np.testing.assert_allclose(out["o"][t, h], 1.3 * ref, rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_exact_retrieval_and_overwrite():
    """gate=1 (log-decay 0), beta=1, orthonormal keys, S0=0: querying k_j (a beta=0 token)
    returns scale*v_j; writing a key again overwrites its value."""
    H, dk, dv, m = 2, 32, 7, 20
    keys = np.stack([np.linalg.qr(RNG.standard_normal((dk, dk)))[0][:, :m].T for _ in range(H)], 1)
    vals = RNG.standard_normal((m, H, dv))
    new1 = RNG.standard_normal((H, dv))
    # m writes, one overwrite of key 3, then m queries
    T = 2 * m + 1
    k = np.zeros((T, H, dk))
    q = RNG.standard_normal((T, H, dk))
    v = np.zeros((T, H, dv))
    beta = np.zeros((T, H))
    k[:m] = keys
    v[:m] = vals
    beta[:m] = 1.0
    k[m] = keys[3]
    v[m] = new1
    beta[m] = 1.0
    q[m + 1:] = keys
    out = _run(q, k, v, np.zeros((T, H, dk)), beta, scale=0.5,
               flags=oracle.GATE_IS_LOG | oracle.NO_QK_L2NORM)
    expect = vals.copy()
    expect[3] = new1
    np.testing.assert_allclose(out["o"][m + 1:], 0.5 * expect, rtol=1e-11, atol=1e-12)


def test_beta_one_self_query_returns_value():
    """beta=1, q_t=k_t, |k_t|=1: S_t^T k_t = v_t for any gates and any S0."""
    T, H, dk, dv = 17, 3, 16, 10
    k = RNG.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = RNG.standard_normal((T, H, dv))
    a = RNG.standard_normal((T, H, dk)) * 2
    S0 = RNG.standard_normal((1, H, dk, dv))
    out = _run(k, k, v, a, np.ones((T, H)), state_in=S0, scale=0.9, flags=oracle.NO_QK_L2NORM)
    np.testing.assert_allclose(out["o"], 0.9 * v, rtol=1e-11, atol=1e-12)


def _brute_force(q, k, v, a, beta, conv_w, conv_b, cs_in, S0, scale, silu):
    """Explicit 128x128 products: S_t = M_t S_{t-1} + beta_t k_t v_t^T with
    M_t = (I - beta_t k_t k_t^T) diag(alpha_t); conv via torch conv1d, gate via scipy."""
    T, H, dk = q.shape
    dv = v.shape[2]
    CC = 2 * H * dk + H * dv
    xall = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], 1)
    y = _conv_lib(xall, conv_w.reshape(CC, 4), conv_b, cs_in, silu)
    qc = y[:, :H * dk].reshape(T, H, dk)
    kc = y[:, H * dk:2 * H * dk].reshape(T, H, dk)
    vc = y[:, 2 * H * dk:].reshape(T, H, dv)
    qn = qc / np.sqrt(np.sum(qc ** 2, -1, keepdims=True) + 1e-6)
    kn = kc / np.sqrt(np.sum(kc ** 2, -1, keepdims=True) + 1e-6)
    alpha = np.exp(-5.0 * scipy.special.expit(a))
    o = np.zeros((T, H, dv))
    Sf = np.zeros((H, dk, dv))
    for h in range(H):
        I = np.eye(dk)
        Ms = [(I - beta[t, h] * np.outer(kn[t, h], kn[t, h])) @ np.diag(alpha[t, h])
              for t in range(T)]
        for t in range(T):
            P = np.eye(dk)
            S = np.zeros((dk, dv))
            # S_t = M_t..M_1 S0 + sum_s M_t..M_{s+1} beta_s k_s v_s^T
            for s in range(t, -1, -1):
                S += P @ (beta[s, h] * np.outer(kn[s, h], vc[s, h]))
                P = P @ Ms[s]
            S += P @ S0[h]
            o[t, h] = scale * S.T @ qn[t, h]
            if t == T - 1:
                Sf[h] = S
    return o, Sf


@pytest.mark.parametrize("T,silu", [(1, False), (2, True), (5, False), (8, False), (8, True)])
def test_brute_force_unrolled_products(T, silu):
    H, dk, dv = 2, 128, 128
    q = RNG.standard_normal((T, H, dk))
    k = RNG.standard_normal((T, H, dk))
    v = RNG.standard_normal((T, H, dv))
    a = RNG.standard_normal((T, H, dk)) * 2
    beta = RNG.random((T, H))
    CC = 2 * H * dk + H * dv
    conv_w = RNG.standard_normal((CC, 4)) * 0.5
    conv_b = RNG.standard_normal(CC) * 0.1
    cs_in = RNG.standard_normal((1, 3, CC))
    S0 = RNG.standard_normal((1, H, dk, dv)) * 0.1
    out = oracle.prefill(q, k, v, a, beta, conv_w, np.array([0, T], np.int32), conv_b=conv_b,
                         conv_state_in=cs_in, state_in=S0, scale=dk ** -0.5,
                         flags=oracle.SILU if silu else 0)
    o_ref, S_ref = _brute_force(q, k, v, a, beta, conv_w, conv_b, cs_in[0], S0[0], dk ** -0.5, silu)
    np.testing.assert_allclose(out["o"], o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["state"][0], S_ref, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------- invariants

def _rand_case(T, H=2, dk=16, dv=12, seed=5):
    r = np.random.default_rng(seed)
    CC = 2 * H * dk + H * dv
    return dict(q=r.standard_normal((T, H, dk)), k=r.standard_normal((T, H, dk)),
                v=r.standard_normal((T, H, dv)), gate=r.standard_normal((T, H, dk)),
                beta=r.random((T, H)), conv_w=r.standard_normal((CC, 4)) * 0.5), \
        r.standard_normal((1, H, dk, dv)) * 0.1, r.standard_normal((1, 3, CC))


def test_homogeneity_in_v_and_state_is_exact():
    c, S0, cs = _rand_case(30)
    cs2 = cs.copy()
    H, dk = c["q"].shape[1], c["q"].shape[2]
    cs2[:, :, 2 * H * dk:] *= 2.0
    cu = np.array([0, 30], np.int32)
    a = oracle.prefill(**c, cu_seqlens=cu, state_in=S0, conv_state_in=cs)
    c2 = dict(c, v=2.0 * c["v"])
    b = oracle.prefill(**c2, cu_seqlens=cu, state_in=2.0 * S0, conv_state_in=cs2)
    np.testing.assert_array_equal(b["o"], 2.0 * a["o"])
    np.testing.assert_array_equal(b["state"], 2.0 * a["state"])


def test_split_prefill_equals_whole():
    c, S0, cs = _rand_case(37)
    whole = oracle.prefill(**c, cu_seqlens=np.array([0, 37], np.int32), state_in=S0,
                           conv_state_in=cs)
    for cut in [1, 2, 3, 20]:
        p1 = {k_: (x[:cut] if k_ != "conv_w" else x) for k_, x in c.items()}
        p2 = {k_: (x[cut:] if k_ != "conv_w" else x) for k_, x in c.items()}
        a = oracle.prefill(**p1, cu_seqlens=np.array([0, cut], np.int32), state_in=S0,
                           conv_state_in=cs)
        b = oracle.prefill(**p2, cu_seqlens=np.array([0, 37 - cut], np.int32),
                           state_in=a["state"], conv_state_in=a["conv_state"])
        np.testing.assert_array_equal(np.concatenate([a["o"], b["o"]]), whole["o"])
        np.testing.assert_array_equal(b["state"], whole["state"])
        np.testing.assert_array_equal(b["conv_state"], whole["conv_state"])


def test_decode_steps_equal_prefill():
    T = 9
    c, S0, cs = _rand_case(T)
    whole = oracle.prefill(**c, cu_seqlens=np.array([0, T], np.int32), state_in=S0,
                           conv_state_in=cs)
    st, conv = S0, cs
    for t in range(T):
        d = oracle.decode(c["q"][t:t + 1], c["k"][t:t + 1], c["v"][t:t + 1], c["gate"][t:t + 1],
                          c["beta"][t:t + 1], c["conv_w"], conv, st)
        np.testing.assert_array_equal(d["o"][0], whole["o"][t])
        st, conv = d["state"], d["conv_state"]
    np.testing.assert_array_equal(st, whole["state"])
    np.testing.assert_array_equal(conv, whole["conv_state"])


def test_varlen_packed_equals_separate_calls():
    lengths = [4, 0, 1, 2, 11]
    T = sum(lengths)
    c, _, _ = _rand_case(T)
    N = len(lengths)
    H, dk, dv = 2, 16, 12
    r = np.random.default_rng(9)
    S0 = r.standard_normal((N, H, dk, dv))
    cs = r.standard_normal((N, 3, 2 * H * dk + H * dv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    packed = oracle.prefill(**c, cu_seqlens=cu, state_in=S0, conv_state_in=cs)
    for n, L in enumerate(lengths):
        s0 = cu[n]
        part = {k_: (x[s0:s0 + L] if k_ != "conv_w" else x) for k_, x in c.items()}
        one = oracle.prefill(**part, cu_seqlens=np.array([0, L], np.int32), state_in=S0[n:n + 1],
                             conv_state_in=cs[n:n + 1])
        np.testing.assert_array_equal(packed["o"][s0:s0 + L], one["o"])
        np.testing.assert_array_equal(packed["state"][n], one["state"][0])
        np.testing.assert_array_equal(packed["conv_state"][n], one["conv_state"][0])
    # an empty sequence passes its state and conv state through unchanged
    np.testing.assert_array_equal(packed["state"][1], S0[1])
    np.testing.assert_array_equal(packed["conv_state"][1], cs[1])


# ----------------------------------------------------- numbers on the pages

def test_state_size_matches_published_arithmetic():
    """The pages state 64 x 128 x 128 = 1,048,576 state scalars per layer, 35,651,584 over
    34 KDA layers, about 136 MiB in FP32 (fixture cites the passage)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "state_size.json")) as f:
        g = json.load(f)
    out = _run(np.zeros((1, g["heads"], g["head_dim"])), np.zeros((1, g["heads"], g["head_dim"])),
               np.zeros((1, g["heads"], g["head_dim"])), np.zeros((1, g["heads"], g["head_dim"])),
               np.zeros((1, g["heads"])))
    per_layer = out["state"][0].size
    assert per_layer == g["state_scalars_per_layer"]
    assert per_layer * g["kda_layers"] == g["state_scalars_per_request"]
    mib = per_layer * g["kda_layers"] * 4 / 2 ** 20
    assert abs(mib - g["fp32_state_mib_approx"]) < 0.5


# -------------------------------------------------------- gate / beta projection

def _proj_inputs(T, hid, H, r=8, dk=4, seed=0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((T, hid)), g.standard_normal((r, hid)) / np.sqrt(hid),
            g.standard_normal((H * dk, r)) / np.sqrt(r), g.standard_normal((H, hid)) / np.sqrt(hid))


def test_gate_proj_zero_weights_give_sigmoid_midpoints():
    x, wa, wb, wbeta = _proj_inputs(5, 16, 3)
    out = oracle.gate_beta_proj(x, 0 * wa, wb, 0 * wbeta, 3, gate_lower_bound=-5.0, log=True)
    assert np.all(out["gate"] == -2.5) and np.all(out["beta"] == 0.5)
    out = oracle.gate_beta_proj(x, wa, 0 * wb, wbeta, 3)
    assert np.all(out["gate"] == 0.0)


def test_gate_proj_brute_force_scalar_loops():
    """Every output against explicit scalar sums on a tiny shape."""
    T, hid, H, r, dk = 3, 6, 2, 4, 3
    x, wa, wb, wbeta = _proj_inputs(T, hid, H, r, dk, seed=1)
    out = oracle.gate_beta_proj(x, wa, wb, wbeta, H, gate_lower_bound=-5.0, log=True)
    for t in range(T):
        z = [sum(wa[i][j] * x[t][j] for j in range(hid)) for i in range(r)]
        for h in range(H):
            for c in range(dk):
                a = sum(wb[h * dk + c][i] * z[i] for i in range(r))
                assert abs(out["gate"][t, h, c] - (-5.0 / (1.0 + math.exp(-a)))) < 1e-12
            b = sum(wbeta[h][j] * x[t][j] for j in range(hid))
            assert abs(out["beta"][t, h] - 1.0 / (1.0 + math.exp(-b))) < 1e-12


def test_gate_proj_selection_weights_closed_form():
    """W_a picks hidden channels 0..r-1, W_b copies z channel (h*dk + c) % r: then
    a[t, h, c] = x[t, (h*dk + c) % r] exactly."""
    T, hid, H, r, dk = 4, 10, 2, 4, 3
    x = np.random.default_rng(2).standard_normal((T, hid))
    wa = np.eye(r, hid)
    wb = np.zeros((H * dk, r))
    for n in range(H * dk):
        wb[n, n % r] = 1.0
    out = oracle.gate_beta_proj(x, wa, wb, np.zeros((H, hid)), H)
    for n in range(H * dk):
        assert np.array_equal(out["gate"].reshape(T, -1)[:, n], x[:, n % r])


def test_gate_proj_beta_sign_symmetry():
    x, wa, wb, wbeta = _proj_inputs(7, 12, 4, seed=3)
    b1 = oracle.gate_beta_proj(x, wa, wb, wbeta, 4)["beta"]
    b2 = oracle.gate_beta_proj(x, wa, wb, -wbeta, 4)["beta"]
    np.testing.assert_allclose(b1 + b2, 1.0, atol=1e-15)
