"""Pins of the oracle's backward pass (gradients of the recurrence; the pages give no backward).

- Central finite differences of the fp64 forward oracle for every input (q, k, v, g, beta, s0),
  on sequences long enough to cross the backward's recomputation checkpoints, with both an
  output and a final-state term in the loss.
- Exact homogeneity: o is linear in q, so <dq, q> = <d_o, o>; (o, S_T) are jointly linear in
  (v, s0), so <dv, v> + <ds0, s0> = L.
- The clamp: the gradient of g is zero where g lies outside [-5, 0].
- Planted mistakes in the backward code are each caught by these checks.
"""
import functools
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


def make_case(seed, lengths=(70, 9), H=2, Dk=4, Dv=3, g_range=(-4.5, -0.3)):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    c = dict(
        q=rng.standard_normal((T, H, Dk)),
        k=rng.standard_normal((T, H, Dk)) / np.sqrt(Dk),
        v=rng.standard_normal((T, H, Dv)),
        g=rng.uniform(*g_range, (T, H, Dk)),
        beta=rng.uniform(0.1, 0.9, (T, H)),
        s0=rng.standard_normal((N, H, Dk, Dv)) * 0.5,
    )
    R1 = rng.standard_normal((T, H, Dv))
    R2 = rng.standard_normal((N, H, Dk, Dv))
    return c, cu, R1, R2


def loss(c, cu, R1, R2, fwd=None):
    o, s = (fwd or oracle.forward)(c["q"], c["k"], c["v"], c["g"], c["beta"], cu, s0=c["s0"])
    return float(np.sum(o * R1) + np.sum(s * R2))


def grads(c, cu, R1, R2, bwd=None):
    return (bwd or oracle.backward)(c["q"], c["k"], c["v"], c["g"], c["beta"], cu, R1, s0=c["s0"], d_sfinal=R2)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "s0": "ds0"}


def check_finite_differences(bwd=None, seed=0, names=tuple(NAMES), samples=40):
    c, cu, R1, R2 = make_case(seed)
    gr = grads(c, cu, R1, R2, bwd)
    rng = np.random.default_rng(seed + 100)
    for name in names:
        x = c[name]
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(samples, flat.size), replace=False)
        fd = np.empty(idx.size)
        for n_, i in enumerate(idx):
            h = 1e-6 * max(1.0, abs(flat[i]))
            old = flat[i]
            flat[i] = old + h
            lp = loss(c, cu, R1, R2)
            flat[i] = old - h
            lm = loss(c, cu, R1, R2)
            flat[i] = old
            fd[n_] = (lp - lm) / (2 * h)
        an = gr[NAMES[name]].reshape(-1)[idx]
        scale = max(np.abs(fd).max(), 1e-3)
        assert np.abs(an - fd).max() <= 2e-6 * scale, (name, np.abs(an - fd).max(), scale)


def check_homogeneity(bwd=None, seed=1):
    c, cu, R1, R2 = make_case(seed, lengths=(100, 37, 1), H=3, Dk=8, Dv=5)
    gr = grads(c, cu, R1, R2, bwd)
    o, s = oracle.forward(c["q"], c["k"], c["v"], c["g"], c["beta"], cu, s0=c["s0"])
    L = np.sum(o * R1) + np.sum(s * R2)
    assert np.sum(gr["dq"] * c["q"]) == pytest.approx(np.sum(o * R1), rel=1e-11, abs=1e-11)
    assert np.sum(gr["dv"] * c["v"]) + np.sum(gr["ds0"] * c["s0"]) == pytest.approx(L, rel=1e-11, abs=1e-11)


def check_clamp_mask(bwd=None, seed=2):
    c, cu, R1, R2 = make_case(seed, g_range=(-7.0, 2.0))
    gr = grads(c, cu, R1, R2, bwd)
    outside = (c["g"] < -5.0) | (c["g"] > 0.0)
    assert outside.any() and (~outside).any()
    assert np.all(gr["dg"][outside] == 0.0)
    assert np.abs(gr["dg"][~outside]).max() > 1e-6


def check_no_final_state_term(bwd=None, seed=3):
    # d_sfinal = None is the same as zeros
    c, cu, R1, R2 = make_case(seed)
    a = (bwd or oracle.backward)(c["q"], c["k"], c["v"], c["g"], c["beta"], cu, R1, s0=c["s0"])
    b = (bwd or oracle.backward)(c["q"], c["k"], c["v"], c["g"], c["beta"], cu, R1, s0=c["s0"],
                                 d_sfinal=np.zeros_like(R2))
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_finite_differences_q_k_v():
    check_finite_differences(names=("q", "k", "v"))


def test_finite_differences_g_beta_s0():
    check_finite_differences(names=("g", "beta", "s0"))


def test_homogeneity():
    check_homogeneity()


def test_clamp_mask():
    check_clamp_mask()


def test_no_final_state_term():
    check_no_final_state_term()


def test_long_sequence_crosses_checkpoints():
    """T = 200 (four checkpoint blocks, the last partial): finite differences on k and g."""
    c, cu, R1, R2 = make_case(4, lengths=(200,), H=1, Dk=3, Dv=2)
    gr = grads(c, cu, R1, R2)
    for name in ("k", "g"):
        flat = c[name].reshape(-1)
        for i in [0, 63 * 3, 64 * 3 + 1, 130 * 3 + 2, flat.size - 1]:
            h = 1e-6
            old = flat[i]
            flat[i] = old + h
            lp = loss(c, cu, R1, R2)
            flat[i] = old - h
            lm = loss(c, cu, R1, R2)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert gr[NAMES[name]].reshape(-1)[i] == pytest.approx(fd, rel=1e-6, abs=1e-8)


# ------------------------------------------------------------------ planted mistakes

BWD_MUTANTS = {
    "no_readout_term": ("dS[i * Dv + j] += qt[i] * dot[j];", ";"),
    "dq_from_previous_state": ("acc += Scur[i * Dv + j] * dot[j];", "acc += Sprev[i * Dv + j] * dot[j];"),
    "dw_sign": ("dw[j] = -bt * du[j];", "dw[j] = bt * du[j];"),
    "no_prediction_term_in_dk": ("dkt[i] += acc;", ";"),
    "dbeta_with_v_only": ("db += du[j] * (vt[j] - w[j]);", "db += du[j] * vt[j];"),
    "dg_without_alpha": ("? da * a[i] : 0.0;", "? da : 0.0;"),
    "clamp_mask_open": ("(gt[i] >= -5.0 && gt[i] <= 0.0)", "(1)"),
    "state_gradient_not_decayed": ("dSt[i * Dv + j] = a[i] * d;", "dSt[i * Dv + j] = d;"),
    "dv_without_beta": ("dvt[j] = bt * du[j];", "dvt[j] = du[j];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = BWD_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    cfile = tmp_path / f"{name}.c"
    cfile.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(cfile), "-o", str(so), "-lm"],
                   check=True)
    bwd = functools.partial(oracle.backward, _lib=oracle.load(str(so)))
    caught = []
    for check in (check_finite_differences, check_homogeneity, check_clamp_mask):
        try:
            check(bwd=bwd)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin catches backward mutant {name}"
