"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle's C source (compiled here, on the CPU) makes at least one pin fail.
The shipped oracle is untouched; mutants live in a temporary directory."""
import ctypes
import os
import subprocess

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "gate_on_dv_axis": ("row[j] *= alpha[i];", "row[j] *= alpha[j];"),
    "no_erase_term": ("u[j] = b * (vt[j] - u[j]);", "u[j] = b * vt[j];"),
    "write_along_q": ("row[j] += kt[i] * u[j];", "row[j] += qt[i] * u[j];"),
    "conv_taps_reversed": ("p - 3 + j,", "p - j,"),
    "gate_sign_flipped": ("gate_lower_bound * sigmoid(a)", "gate_lower_bound * sigmoid(-a)"),
    "k_normalised_by_q_norm": ("kt[c] *= ik;", "kt[c] *= iq;"),
    "scale_dropped": ("scale * ot[j]", "ot[j]"),
    "eps_outside_root": ("sqrt(sq + L2_EPS)", "(sqrt(sq) + L2_EPS)"),
    "beta_dropped": ("u[j] = b * (vt[j] - u[j]);", "u[j] = (vt[j] - u[j]);"),
}

# the fast pins, by name, from the pin module
PINS = [
    "test_short_conv_matches_torch_conv1d",
    "test_l2_norm_closed_form",
    "test_gate_sigmoid_values_and_row_axis",
    "test_beta_zero_is_pure_gated_decay",
    "test_one_hot_keys_reduce_to_gla",
    "test_orthonormal_keys_exact_retrieval_and_overwrite",
    "test_beta_one_self_query_returns_value",
    "test_brute_force_unrolled_products",
]


def _run_pins():
    from tests import test_oracle_pins as P
    failed = []
    for name in PINS:
        fn = getattr(P, name)
        try:
            if name == "test_short_conv_matches_torch_conv1d":
                fn(False, True)
            elif name == "test_brute_force_unrolled_products":
                fn(5, False)
            else:
                fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path, monkeypatch):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor missing: " + old
    mpath = tmp_path / "mut.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    str(mpath), "-o", str(so), "-lm"], check=True)
    lib = oracle._bind(ctypes.CDLL(str(so)))
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = _run_pins()
    assert failed, "no pin caught mutant " + mutant


def test_unmutated_oracle_passes_the_same_pins():
    assert _run_pins() == []


# --------------------------------------------- the projection oracle (Python)

PROJ_MUTANTS = {
    "gate_sigmoid_sign_flipped": ("gate_lower_bound * sig(a)", "gate_lower_bound * sig(-a)"),
    "gate_bound_dropped": ("gate_lower_bound * sig(a)", "sig(a)"),
    "beta_without_sigmoid": ("beta = sig(x @ w_beta.T)", "beta = x @ w_beta.T"),
    "head_and_channel_swapped": ('gate.reshape(T, num_heads, -1)',
                                 'gate.reshape(T, -1, num_heads).transpose(0, 2, 1)'),
    "second_factor_dropped": ("a = z @ w_b.T", "a = z @ np.eye(z.shape[1], w_b.shape[0])"),
}

PROJ_PINS = ["test_gate_proj_zero_weights_give_sigmoid_midpoints",
             "test_gate_proj_brute_force_scalar_loops",
             "test_gate_proj_selection_weights_closed_form",
             "test_gate_proj_beta_sign_symmetry"]


@pytest.mark.parametrize("mutant", sorted(PROJ_MUTANTS))
def test_planted_projection_mistake_is_caught(mutant, monkeypatch):
    import inspect
    import textwrap
    import numpy as np
    from tests import test_oracle_pins as P
    old, new = PROJ_MUTANTS[mutant]
    src = textwrap.dedent(inspect.getsource(oracle.gate_beta_proj))
    assert src.count(old) == 1, "mutation anchor missing: " + old
    ns = {"np": np, "_f64": oracle._f64}
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "gate_beta_proj", ns["gate_beta_proj"])
    caught = []
    for name in PROJ_PINS:
        try:
            getattr(P, name)()
        except (AssertionError, ValueError):
            caught.append(name)
    assert caught, "no pin catches " + mutant


def test_projection_harness_control(monkeypatch):
    """The same path with the source unchanged: every pin passes."""
    import inspect
    import textwrap
    import numpy as np
    from tests import test_oracle_pins as P
    ns = {"np": np, "_f64": oracle._f64}
    exec(textwrap.dedent(inspect.getsource(oracle.gate_beta_proj)), ns)
    monkeypatch.setattr(oracle, "gate_beta_proj", ns["gate_beta_proj"])
    for name in PROJ_PINS:
        getattr(P, name)()
