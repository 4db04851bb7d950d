"""Pins of the oracle's input prologue (gate logits, beta logits, unit q/k).

The pages fix only the roles of alpha and beta and the clamp of alpha to
[e^-5, 1]; the logit forms are the customary parameterisation and are pinned
here by what mathematics fixes about them: closed-form values (softplus(0) =
ln 2, softplus(ln(e^c - 1)) = c, sigmoid(ln(p / (1 - p))) = p), symmetries
(softplus(x) - softplus(-x) = x, sigmoid(x) + sigmoid(-x) = 1, softplus' =
sigmoid), a Pythagorean unit vector, and end-to-end reductions of the
recurrence to runs with known gates (alpha = 1/2, alpha = 1, the lower clamp,
beta = 1/2, beta = 1 with the delta-rule identity o_t = v_t).
"""
import math

import numpy as np
import pytest

import kda_inputs
import oracle


def test_softplus_closed_forms():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    for c in [1e-3, 0.5, 1.0, 3.0, 10.0, 30.0]:
        x = math.log(math.expm1(c))  # ln(e^c - 1)
        assert oracle.softplus(x) == pytest.approx(c, rel=1e-13)
    # no overflow at either end
    assert oracle.softplus(800.0) == 800.0
    assert 0.0 <= oracle.softplus(-800.0) < 1e-300


def test_softplus_symmetry_and_derivative():
    x = np.linspace(-40, 40, 801)
    np.testing.assert_allclose(oracle.softplus(x) - oracle.softplus(-x), x, rtol=0, atol=1e-13)
    h = 1e-5
    d = (oracle.softplus(x + h) - oracle.softplus(x - h)) / (2 * h)
    np.testing.assert_allclose(d, oracle.sigmoid(x), rtol=0, atol=1e-9)


def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    for p in [1e-6, 0.1, 0.25, 0.9, 0.999]:
        assert oracle.sigmoid(math.log(p / (1 - p))) == pytest.approx(p, rel=1e-12)
    x = np.linspace(-50, 50, 1001)
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert oracle.sigmoid(-800.0) == 0.0 and oracle.sigmoid(800.0) == 1.0
    assert oracle.sigmoid(40.0) == 1.0  # 1 - 4e-18 rounds to 1 in fp64


def test_unit_rows():
    np.testing.assert_array_equal(oracle.unit_rows(np.array([3.0, 4.0])), [0.6, 0.8])
    np.testing.assert_array_equal(oracle.unit_rows(np.zeros((2, 5))), np.zeros((2, 5)))
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 128)) * rng.uniform(0.01, 100, (50, 3, 1))
    u = oracle.unit_rows(x)
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=1e-14)
    # parallel and with the same orientation: <x, u> = ||x||
    np.testing.assert_allclose(np.sum(x * u, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def _case(rng, T=40, H=2, Dk=8, Dv=6):
    q = rng.standard_normal((T, H, Dk))
    k = rng.standard_normal((T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, Dv))
    beta = rng.uniform(0, 1, (T, H))
    s0 = rng.standard_normal((1, H, Dk, Dv)) * 0.3
    return q, k, v, beta, s0


def _fwd(q, k, v, g, beta, s0, **flags):
    q, k, g, beta = oracle.prologue(q, k, g, beta, **flags)
    return oracle.forward(q, k, v, g, beta, np.array([0, q.shape[0]]), s0=s0)


def test_gate_logit_zero_is_half_forget():
    rng = np.random.default_rng(1)
    q, k, v, beta, s0 = _case(rng)
    g0 = np.zeros(q.shape)
    o1, s1 = _fwd(q, k, v, g0, beta, s0, g_logit=True)
    o2, s2 = _fwd(q, k, v, np.full(q.shape, -math.log(2.0)), beta, s0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-14)


def test_gate_logit_far_negative_keeps_state():
    rng = np.random.default_rng(2)
    q, k, v, beta, s0 = _case(rng)
    o1, s1 = _fwd(q, k, v, np.full(q.shape, -60.0), beta, s0, g_logit=True)
    o2, s2 = _fwd(q, k, v, np.zeros(q.shape), beta, s0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-12)


def test_gate_logit_large_hits_lower_clamp():
    # log alpha = -softplus(10) = -10.0000454, clamped to -5
    rng = np.random.default_rng(3)
    q, k, v, beta, s0 = _case(rng)
    o1, s1 = _fwd(q, k, v, np.full(q.shape, 10.0), beta, s0, g_logit=True)
    o2, s2 = _fwd(q, k, v, np.full(q.shape, -5.0), beta, s0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_beta_logit_zero_is_half():
    rng = np.random.default_rng(4)
    q, k, v, _, s0 = _case(rng)
    g = -oracle.softplus(rng.standard_normal(q.shape))
    o1, s1 = _fwd(q, k, v, g, np.zeros(q.shape[:2]), s0, beta_logit=True)
    o2, s2 = _fwd(q, k, v, g, np.full(q.shape[:2], 0.5), s0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_unnormalised_keys_with_l2norm_keep_the_delta_identity():
    # beta = sigmoid(40) = 1 and q = k scaled to unit length: every token reads back its own value
    rng = np.random.default_rng(5)
    T, H, Dk, Dv = 30, 2, 16, 5
    k = rng.standard_normal((T, H, Dk)) * rng.uniform(0.1, 10, (T, H, 1))
    v = rng.standard_normal((T, H, Dv))
    g = rng.standard_normal((T, H, Dk))
    o, _ = _fwd(k * 3.0, k, v, g, np.full((T, H), 40.0), rng.standard_normal((1, H, Dk, Dv)),
                g_logit=True, beta_logit=True, qk_l2norm=True)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_l2norm_removes_the_scale_of_q_and_k():
    rng = np.random.default_rng(6)
    q, k, v, beta, s0 = _case(rng)
    g = rng.standard_normal(q.shape)
    o1, s1 = _fwd(q, k, v, g, beta, s0, g_logit=True, qk_l2norm=True)
    cq = rng.uniform(0.01, 50, q.shape[:2] + (1,))
    ck = rng.uniform(0.01, 50, q.shape[:2] + (1,))
    o2, s2 = _fwd(q * cq, k * ck, v, g, beta, s0, g_logit=True, qk_l2norm=True)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=0, atol=1e-12)
    # and without the norm the scale does change the result
    o3, _ = _fwd(q * cq, k * ck, v, g, beta, s0, g_logit=True)
    assert np.abs(o3 - o1).max() > 1e-3


def test_l2norm_zero_rows_stay_zero():
    rng = np.random.default_rng(7)
    q, k, v, beta, s0 = _case(rng)
    q[3] = 0.0
    k[5] = 0.0
    g = -oracle.softplus(rng.standard_normal(q.shape))
    o1, s1 = _fwd(q, k, v, g, beta, s0, qk_l2norm=True)
    assert np.all(o1[3] == 0.0)
    # a zero key writes nothing and erases nothing: same as beta = 0 for that token
    b2 = beta.copy()
    b2[5] = 0.0
    kk = k.copy()
    kk[5] = 1.0  # any key; beta = 0 removes it
    o2, s2 = _fwd(q, kk, v, g, b2, s0, qk_l2norm=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-13)


def test_generator_raw_forms_map_to_the_default_inputs():
    # the generator draws gate and beta logits from the same streams as the default
    # inputs; after the prologue both describe the same gates (the defaults were rounded
    # to float32 by the generator)
    base = dict(lengths=[70], H=2, Dk=64, Dv=64, dtype="f32", gate="softplus", seed=11)
    a = kda_inputs.generate(kda_inputs.Spec(**base))
    b = kda_inputs.generate(kda_inputs.Spec(**base, g_logit=True, beta_logit=True))
    _, _, g, beta = oracle.prologue(b.q, b.k, b.g, b.beta, g_logit=True, beta_logit=True)
    np.testing.assert_allclose(g, a.g, rtol=1e-6, atol=0)
    np.testing.assert_allclose(beta, a.beta, rtol=1e-6, atol=0)


def test_generator_bf16_gates_are_bf16_bits():
    sp = kda_inputs.Spec([65], 1, 64, 64, "bf16", "softplus", seed=3, gate_dtype="bf16", g_logit=True)
    inp = kda_inputs.generate(sp)
    assert inp.g.dtype == np.uint16 and inp.beta.dtype == np.uint16
    f = inp.as_f32("g")
    assert np.all(f.view(np.uint32) & 0xFFFF == 0)


# ------------------------------------------------------------------ planted mistakes

CHECKS = [test_softplus_closed_forms, test_softplus_symmetry_and_derivative, test_sigmoid_closed_forms,
          test_unit_rows, test_gate_logit_zero_is_half_forget, test_gate_logit_far_negative_keeps_state,
          test_gate_logit_large_hits_lower_clamp, test_beta_logit_zero_is_half,
          test_unnormalised_keys_with_l2norm_keep_the_delta_identity, test_l2norm_removes_the_scale_of_q_and_k,
          test_l2norm_zero_rows_stay_zero]

_sp, _sg, _ur = oracle.softplus, oracle.sigmoid, oracle.unit_rows
PROLOGUE_MUTANTS = {
    "softplus_sign_inside": ("softplus", lambda x: np.maximum(x, 0.0) + np.log1p(np.exp(np.abs(x)))),
    "softplus_no_max_term": ("softplus", lambda x: np.log1p(np.exp(-np.abs(np.asarray(x, float))))),
    "softplus_log_not_log1p": ("softplus", lambda x: np.maximum(x, 0.0) + np.log(np.exp(-np.abs(x)))),
    "softplus_is_relu": ("softplus", lambda x: np.maximum(np.asarray(x, float), 0.0)),
    "sigmoid_flipped": ("sigmoid", lambda x: _sg(-np.asarray(x, float))),
    "sigmoid_is_tanh": ("sigmoid", lambda x: np.tanh(np.asarray(x, float))),
    "unit_rows_noop": ("unit_rows", lambda x: np.asarray(x, float)),
    "unit_rows_squared_norm": ("unit_rows", lambda x: np.asarray(x, float) / np.maximum(
        np.sum(np.asarray(x, float) ** 2, axis=-1, keepdims=True), 1e-300)),
    "unit_rows_l1": ("unit_rows", lambda x: np.asarray(x, float) / np.maximum(
        np.sum(np.abs(np.asarray(x, float)), axis=-1, keepdims=True), 1e-300)),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTANTS))
def test_prologue_mutant_is_caught(name, monkeypatch):
    attr, fn = PROLOGUE_MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for check in CHECKS:
            try:
                check()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(check.__name__)
    assert caught, f"no prologue pin catches {name}"
