"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each check targets a different class of mistake: the hand-worked example and
exact rational arithmetic fix every operation; the dense unrolled product fixes
the order of forget / erase / write; the scalar closed form fixes the first-order
recurrence; the clamp checks fix the gate bounds printed on the worldcybernews
page (second paragraph); invariants (zero in / zero out, alpha=1 & beta=0,
beta=1 with unit keys, orthonormal keys) and structural properties (linearity,
column independence, key permutation, split/resume, varlen) fix the rest.
``test_oracle_mutants.py`` shows that planted mistakes in the oracle fail these.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(q, k, v, g, beta, cu=None, s0=None, cols=None, fwd=None):
    fwd = fwd or oracle.forward
    total = q.shape[0]
    if cu is None:
        cu = np.array([0, total], dtype=np.int64)
    return fwd(q, k, v, g, beta, cu, s0=s0, cols=cols)


def rand_case(rng, T, H, Dk, Dv, unit_keys=True, s0=True, N=1):
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    k = rng.standard_normal((T, H, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    g = (-np.logaddexp(0, rng.standard_normal((T, H, Dk)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    S0 = rng.standard_normal((N, H, Dk, Dv)) * 0.3 if s0 else None
    return q, k, v, g, beta, S0


# ------------------------------------------------------------------ worked example

def check_worked_example(fwd=None):
    d = json.load(open(os.path.join(GOLDEN, "worked_d2_t2.json")))
    toks = d["tokens"]
    F = lambda x: float(Fraction(str(x)))
    q = np.array([[[F(x) for x in t["q"]]] for t in toks], dtype=np.float32)
    k = np.array([[[F(x) for x in t["k"]]] for t in toks], dtype=np.float32)
    v = np.array([[[F(x) for x in t["v"]]] for t in toks], dtype=np.float32)
    g = np.array([[[math.log(F(a)) for a in t["alpha"]]] for t in toks], dtype=np.float32)
    beta = np.array([[t["beta"]] for t in toks], dtype=np.float32)
    o, S = run(q, k, v, g, beta, fwd=fwd)
    o_exp = np.array([[F(x) for x in row] for row in d["expected"]["o"]])
    S_exp = np.array([[F(x) for x in row] for row in d["expected"]["S_final"]])
    np.testing.assert_allclose(o[:, 0, :], o_exp, rtol=0, atol=3e-7)
    np.testing.assert_allclose(S[0, 0], S_exp, rtol=0, atol=3e-7)


def test_worked_example():
    check_worked_example()


# ------------------------------------------------------------------ exact rationals

def exact_matrix_recurrence(q, k, v, g, beta, S0):
    """S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T in exact rationals (matrix form)."""
    T, Dk = q.shape
    Dv = v.shape[1]
    Fr = lambda x: Fraction(float(x))
    S = [[Fr(S0[i, j]) for j in range(Dv)] for i in range(Dk)]
    outs = []
    for t in range(T):
        a = [Fraction(math.exp(min(0.0, max(-5.0, float(g[t, i]))))) for i in range(Dk)]
        kk = [Fr(x) for x in k[t]]
        b = Fr(beta[t])
        A = [[(Fraction(int(i == j)) - b * kk[i] * kk[j]) * a[j] for j in range(Dk)] for i in range(Dk)]
        S = [[sum(A[i][m] * S[m][j] for m in range(Dk)) + b * kk[i] * Fr(v[t, j]) for j in range(Dv)]
             for i in range(Dk)]
        qq = [Fr(x) for x in q[t]]
        outs.append([sum(S[i][j] * qq[i] for i in range(Dk)) for j in range(Dv)])
    return outs, S


def check_exact_rationals(fwd=None, seeds=range(4)):
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        T, Dk, Dv = 6 + seed % 3, 3 + seed % 2, 2 + seed % 3
        q, k, v, g, beta, S0 = rand_case(rng, T, 1, Dk, Dv)
        # a few gates exactly at / beyond the clamp bounds and at alpha = 1
        g[0, 0, 0] = -5.0
        g[1, 0, -1] = 0.0
        g[2, 0, 0] = -6.5
        g[3, 0, 1 % Dk] = 0.75
        o, S = run(q, k, v, g, beta, s0=S0, fwd=fwd)
        outs, S_ex = exact_matrix_recurrence(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0[0, 0])
        o_ex = np.array([[float(x) for x in row] for row in outs])
        S_exf = np.array([[float(x) for x in row] for row in S_ex])
        scale = max(1.0, np.abs(o_ex).max())
        assert np.abs(o[:, 0, :] - o_ex).max() <= 1e-13 * scale, f"seed {seed}"
        assert np.abs(S[0, 0] - S_exf).max() <= 1e-13 * max(1.0, np.abs(S_exf).max()), f"seed {seed}"


def test_exact_rationals():
    check_exact_rationals()


# ------------------------------------------------------------------ dense brute force

def dense_unrolled(q, k, v, g, beta, S0):
    """S_T = prod_{r=T..1} A_r S0 + sum_s (prod_{r=T..s+1} A_r) b_s k_s v_s^T with dense A_r;
    o_t taken from S_t built the same unrolled way (no running state)."""
    T, Dk = q.shape
    alpha = np.exp(np.clip(g.astype(np.float64), -5, 0))
    A = [(np.eye(Dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(alpha[t]) for t in range(T)]
    Bw = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    outs = []
    for t in range(T):
        # product A_t ... A_0 applied to S0
        M = np.eye(Dk)
        for r in range(0, t + 1):
            M = A[r] @ M
        St = M @ S0
        for s in range(t + 1):
            Pm = np.eye(Dk)
            for r in range(s + 1, t + 1):
                Pm = A[r] @ Pm
            St = St + Pm @ Bw[s]
        outs.append(St.T @ q[t])
    return np.array(outs), St


def check_dense_bruteforce(fwd=None):
    for seed in range(6):
        rng = np.random.default_rng(seed)
        T = 1 + seed + (seed > 3)  # 1..8
        Dk, Dv = (4, 3) if seed % 2 else (5, 5)
        q, k, v, g, beta, S0 = rand_case(rng, T, 1, Dk, Dv, unit_keys=bool(seed % 3))
        o, S = run(q, k, v, g, beta, s0=S0, fwd=fwd)
        f64 = lambda a: a[:, 0].astype(np.float64)
        o_ref, S_ref = dense_unrolled(f64(q), f64(k), f64(v), f64(g), beta[:, 0].astype(np.float64), S0[0, 0])
        np.testing.assert_allclose(o[:, 0], o_ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(S[0, 0], S_ref, rtol=1e-13, atol=1e-13)


def test_dense_bruteforce():
    check_dense_bruteforce()


# ------------------------------------------------------------------ scalar closed form

def check_scalar_closed_form(fwd=None):
    """d_k = d_v = 1: s_t = a_t s_{t-1} + b_t with a_t = (1 - beta k^2) alpha, b_t = beta k v,
    whose solution is s_T = (prod a) s_0 + sum_t (prod_{r>t} a_r) b_t."""
    rng = np.random.default_rng(7)
    T = 40
    q, k, v, g, beta, S0 = rand_case(rng, T, 1, 1, 1, unit_keys=False)
    k = (k * 0.9).astype(np.float32)
    o, S = run(q, k, v, g, beta, s0=S0, fwd=fwd)
    a = (1 - beta[:, 0].astype(np.float64) * k[:, 0, 0].astype(np.float64) ** 2) * np.exp(
        np.clip(g[:, 0, 0].astype(np.float64), -5, 0))
    b = beta[:, 0].astype(np.float64) * k[:, 0, 0] * v[:, 0, 0]
    outs = []
    for t in range(T):
        st = np.prod(a[: t + 1]) * S0[0, 0, 0, 0] + sum(np.prod(a[s + 1: t + 1]) * b[s] for s in range(t + 1))
        outs.append(st * q[t, 0, 0])
        if t == T - 1:
            np.testing.assert_allclose(S[0, 0, 0, 0], st, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o[:, 0, 0], np.array(outs), rtol=1e-12, atol=1e-14)


def test_scalar_closed_form():
    check_scalar_closed_form()


# ------------------------------------------------------------------ invariants

def check_identity_gate(fwd=None):
    """alpha = 1 (g = 0) and beta = 0: the state never changes and o_t = S0^T q_t."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = rand_case(rng, 20, 2, 6, 5)
    g[:] = 0.0
    beta[:] = 0.0
    o, S = run(q, k, v, g, beta, s0=S0, fwd=fwd)
    assert np.array_equal(S, S0)
    o_ref = np.einsum("hij,thi->thj", S0[0], q.astype(np.float64))
    np.testing.assert_allclose(o, o_ref, rtol=1e-14, atol=1e-14)


def test_identity_gate():
    check_identity_gate()


def check_unit_key_write(fwd=None):
    """beta = 1 and a unit key: k_t^T S_t = v_t^T for any alpha; with q_t = k_t, o_t = v_t."""
    rng = np.random.default_rng(4)
    T, Dk, Dv = 30, 8, 6
    k = rng.standard_normal((T, 1, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    q = k.copy()
    v = rng.standard_normal((T, 1, Dv)).astype(np.float32)
    g = (-rng.uniform(0, 6, (T, 1, Dk))).astype(np.float32)
    beta = np.ones((T, 1), dtype=np.float32)
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    o, S = run(q, k, v, g, beta, s0=S0, fwd=fwd)
    # float32 keys are unit only to ~1e-7; the identity holds to that order
    kn2 = (k.astype(np.float64) ** 2).sum(-1)
    assert np.abs(kn2 - 1).max() < 1e-6
    np.testing.assert_allclose(o[:, 0], v[:, 0].astype(np.float64), rtol=0, atol=1e-5)
    np.testing.assert_allclose(k[-1, 0].astype(np.float64) @ S[0, 0], v[-1, 0], rtol=0, atol=1e-5)
    # exactly unit keys (coordinate axes): the identity is exact up to fp64 rounding
    idx = rng.integers(0, Dk, T)
    k2 = np.zeros((T, 1, Dk), dtype=np.float32)
    k2[np.arange(T), 0, idx] = 1.0
    o2, S2 = run(k2, k2, v, g, beta, s0=S0, fwd=fwd)
    np.testing.assert_allclose(o2[:, 0], v[:, 0].astype(np.float64), rtol=0, atol=1e-15)


def test_unit_key_write():
    check_unit_key_write()


def check_zero(fwd=None):
    rng = np.random.default_rng(5)
    q, k, v, g, beta, _ = rand_case(rng, 17, 2, 4, 4, s0=False)
    z = np.zeros_like
    o, S = run(z(q), z(k), z(v), g, beta, fwd=fwd)
    assert not o.any() and not S.any()
    # zero keys and values with a random gate: still nothing is written
    o, S = run(q, z(k), z(v), g, beta, fwd=fwd)
    assert not o.any() and not S.any()


def test_zero_in_zero_out():
    check_zero()


def check_orthonormal_keys(fwd=None):
    """alpha = 1, beta = 1, S0 = 0, orthonormal keys: S_T = sum_s k_s v_s^T and o_t = v_s
    when q_t = k_s with s <= t, else 0."""
    rng = np.random.default_rng(6)
    Dk, Dv, T = 8, 5, 8
    perm = rng.permutation(Dk)
    # keys that are exactly orthonormal in float32: signed coordinate axes
    k = np.zeros((T, 1, Dk))
    k[np.arange(T), 0, perm] = rng.choice([-1.0, 1.0], T)
    k = k.astype(np.float32)
    v = rng.standard_normal((T, 1, Dv)).astype(np.float32)
    g = np.zeros((T, 1, Dk), dtype=np.float32)
    beta = np.ones((T, 1), dtype=np.float32)
    qsel = rng.integers(0, T, T)
    q = k[qsel].copy()
    o, S = run(q, k, v, g, beta, fwd=fwd)
    S_ref = sum(np.outer(k[s, 0], v[s, 0]) for s in range(T))
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=0, atol=1e-15)
    for t in range(T):
        s = qsel[t]
        exp_o = v[s, 0] if s <= t else np.zeros(Dv)
        np.testing.assert_allclose(o[t, 0], exp_o, rtol=0, atol=1e-15)


def test_orthonormal_keys():
    check_orthonormal_keys()


def check_clamp(fwd=None):
    """The forget gate is clamped to [e^-5, 1]: g below -5 acts as -5, g above 0 acts as 0."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, S0 = rand_case(rng, 12, 1, 4, 3)
    g_lo = g.copy()
    g_lo[::2] = -5.0
    g_lo[1::2] = 0.0
    g_out = g_lo.copy()
    g_out[::2] = -9.0
    g_out[1::2] = 2.5
    g_inf = g_lo.copy()
    g_inf[::2] = -np.inf
    g_inf[1::2] = np.inf
    a, sa = run(q, k, v, g_lo, beta, s0=S0, fwd=fwd)
    b, sb = run(q, k, v, g_out, beta, s0=S0, fwd=fwd)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
    c, sc = run(q, k, v, g_inf, beta, s0=S0, fwd=fwd)  # infinite logs of alpha sit at the bounds too
    assert np.array_equal(a, c) and np.array_equal(sa, sc)
    # the lower bound is e^-5 itself: one token, beta = 0, S0 = I-like -> S = e^-5 S0
    z1 = np.zeros((1, 1, 4), dtype=np.float32)
    S0i = np.eye(4)[None, None, :, :3].copy()
    _, s = run(z1, z1, np.zeros((1, 1, 3), np.float32), np.full((1, 1, 4), -50, np.float32),
               np.zeros((1, 1), np.float32), s0=S0i, fwd=fwd)
    np.testing.assert_allclose(s[0, 0], math.exp(-5) * S0i[0, 0], rtol=1e-15, atol=0)
    _, s = run(z1, z1, np.zeros((1, 1, 3), np.float32), np.full((1, 1, 4), 3.0, np.float32),
               np.zeros((1, 1), np.float32), s0=S0i, fwd=fwd)
    assert np.array_equal(s[0, 0], S0i[0, 0])


def test_clamp_bounds():
    check_clamp()


# ------------------------------------------------------------------ structure

def check_linearity(fwd=None):
    """o and S_T are jointly linear in (V, S0) for fixed q, k, g, beta."""
    rng = np.random.default_rng(9)
    q, k, v1, g, beta, S01 = rand_case(rng, 25, 2, 6, 4)
    # values on a 2^-8 grid so that a*v1 + b*v2 is exact in float32
    v1 = (np.round(v1 * 256) / 256).astype(np.float32)
    v2 = (np.round(rng.standard_normal(v1.shape) * 256) / 256).astype(np.float32)
    S02 = rng.standard_normal(S01.shape)
    a, b = 0.75, -1.25
    o1, s1 = run(q, k, v1, g, beta, s0=S01, fwd=fwd)
    o2, s2 = run(q, k, v2, g, beta, s0=S02, fwd=fwd)
    v3 = (a * v1.astype(np.float64) + b * v2).astype(np.float32)  # exact: dyadic scalars
    assert np.array_equal(v3.astype(np.float64), a * v1.astype(np.float64) + b * v2)
    o3, s3 = run(q, k, v3, g, beta, s0=a * S01 + b * S02, fwd=fwd)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + b * s2, rtol=1e-12, atol=1e-12)


def test_linearity():
    check_linearity()


def check_columns(fwd=None):
    """Columns of S are independent: a subset / permutation of d_v columns gives the same
    numbers, bit for bit, and permuting v's channels permutes o's and S's columns."""
    rng = np.random.default_rng(10)
    q, k, v, g, beta, S0 = rand_case(rng, 33, 2, 8, 20)
    o, s = run(q, k, v, g, beta, s0=S0, fwd=fwd)
    cols = [19, 3, 3, 0, 7]
    oc, sc = run(q, k, v, g, beta, s0=S0, cols=cols, fwd=fwd)
    assert np.array_equal(oc, o[:, :, cols]) and np.array_equal(sc, s[..., cols])
    perm = rng.permutation(20)
    op, sp = run(q, k, v[:, :, perm], g, beta, s0=S0[..., perm], fwd=fwd)
    assert np.array_equal(op, o[:, :, perm]) and np.array_equal(sp, s[..., perm])


def test_column_independence():
    check_columns()


def check_key_permutation(fwd=None):
    """Permuting d_k channels jointly in q, k, g and the rows of S0 leaves o unchanged."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rand_case(rng, 30, 1, 7, 3)
    o, s = run(q, k, v, g, beta, s0=S0, fwd=fwd)
    p = rng.permutation(7)
    op, sp = run(q[..., p], k[..., p], v, g[..., p], beta, s0=S0[:, :, p, :], fwd=fwd)
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sp, s[:, :, p, :], rtol=1e-12, atol=1e-12)


def test_key_permutation():
    check_key_permutation()


def check_split_resume(fwd=None):
    """Running [0, T1) and then [T1, T) from the carried state equals the unbroken run."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = rand_case(rng, 50, 2, 6, 5)
    o, s = run(q, k, v, g, beta, s0=S0, fwd=fwd)
    for T1 in (0, 1, 23, 49, 50):
        oa, sa = run(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], s0=S0, fwd=fwd)
        ob, sb = run(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], s0=sa, fwd=fwd)
        assert np.array_equal(np.concatenate([oa, ob]), o) and np.array_equal(sb, s)


def test_split_resume():
    check_split_resume()


def check_varlen(fwd=None):
    """Packed sequences equal separate calls; empty sequences pass S0 through."""
    rng = np.random.default_rng(13)
    lens = [5, 0, 17, 1, 9]
    T = sum(lens)
    q, k, v, g, beta, S0 = rand_case(rng, T, 2, 4, 3, N=len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    o, s = run(q, k, v, g, beta, cu=cu, s0=S0, fwd=fwd)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, sn = run(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0=S0[n:n + 1], fwd=fwd)
        assert np.array_equal(on, o[a:b]) and np.array_equal(sn[0], s[n])
    assert np.array_equal(s[1], S0[1])


def test_varlen_equals_separate():
    check_varlen()


def check_nonexpansion(fwd=None):
    """With unit keys, beta in [0, 1] and alpha <= 1, (I - beta k k^T) and Diag(alpha) are
    contractions, so ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = rand_case(rng, 40, 1, 6, 4)
    k = k.astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    prev = np.linalg.norm(S0[0, 0])
    S = S0
    for t in range(40):
        _, S = run(q[t:t + 1], k[t:t + 1].astype(np.float32), v[t:t + 1], g[t:t + 1], beta[t:t + 1], s0=S,
                   fwd=fwd)
        cur = np.linalg.norm(S[0, 0])
        assert cur <= prev + beta[t, 0] * np.linalg.norm(v[t, 0].astype(np.float64)) + 1e-6
        prev = cur


def test_nonexpansion():
    check_nonexpansion()


ALL_CHECKS = [check_worked_example, check_exact_rationals, check_dense_bruteforce, check_scalar_closed_form,
              check_identity_gate, check_unit_key_write, check_zero, check_orthonormal_keys, check_clamp,
              check_linearity, check_columns, check_key_permutation, check_split_resume, check_varlen,
              check_nonexpansion]
