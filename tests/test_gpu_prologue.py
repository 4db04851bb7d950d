"""GPU parity of the input prologue (gate logits, beta logits, bf16 gates, unit q/k inside the
kernels) against the oracle with its fp64 prologue, on every entry point and both prefill paths."""
import numpy as np
import pytest
import torch

import gated_delta_rule_65_amd as kda
import kda_inputs
import oracle
from tests.gpu_util import TOL, rel_err, to_dev
from tests.test_gpu_decode import run_decode
from tests.test_gpu_parity import PATHS, check, run_chunk

pytestmark = pytest.mark.gpu

ALL = dict(g_logit=True, beta_logit=True, qk_l2norm=True)


@PATHS
@pytest.mark.parametrize("flags", [
    dict(), dict(g_logit=True), dict(beta_logit=True), dict(qk_l2norm=True), ALL,
], ids=["bf16_gates_only", "g_logit", "beta_logit", "qk_l2norm", "all"])
def test_chunk_prologue_bf16_gates(flags, fused):
    spec = kda_inputs.Spec([200] * 2, 3, 128, 128, "bf16", "softplus", s0_std=0.02, seed=61, gate_dtype="bf16",
                           name="pro-" + "-".join(sorted(flags)), **flags)
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128)])
def test_chunk_prologue_f32(Dk, Dv, fused):
    spec = kda_inputs.Spec([150] * 2, 2, Dk, Dv, "f32", "softplus", s0_std=0.1, seed=62, name=f"pro-f32-{Dk}",
                           **ALL)
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
def test_chunk_prologue_wide_logits_hit_both_bounds(fused):
    """logits ~ N(0, 4^2): many gates clamp at log alpha = -5, many sit near alpha = 1."""
    spec = kda_inputs.Spec([333], 4, 128, 128, "bf16", "softplus", seed=63, logit_std=4.0, name="pro-wide",
                           **ALL)
    inp = kda_inputs.generate(spec)
    g = oracle.prologue(inp.q[:1], inp.k[:1], inp.as_f32("g"), inp.beta[:1], g_logit=True)[2]
    assert (g <= -5).mean() > 0.05 and (g > -0.01).mean() > 0.05
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
def test_varlen_prologue(fused):
    spec = kda_inputs.Spec([0, 1, 64, 65, 190, 7], 3, 128, 128, "bf16", "softplus", s0_std=0.02, seed=64,
                           packed=True, gate_dtype="bf16", name="pro-varlen", **ALL)
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, batched=False, fused=fused))


@PATHS
def test_l2norm_zero_rows_and_scale_invariance(fused):
    spec = kda_inputs.Spec([130] * 2, 2, 128, 128, "f32", "softplus", s0_std=0.1, seed=65, name="pro-zero", **ALL)
    inp = kda_inputs.generate(spec)
    inp.q[5] = 0.0
    inp.k[70] = 0.0
    o, s = run_chunk(inp, fused=fused)
    check(inp, o, s)
    assert not o[5].any()
    # scaling q and k rows by positive factors changes nothing beyond rounding
    rng = np.random.default_rng(0)
    inp.q *= rng.uniform(0.05, 20, inp.q.shape[:2] + (1,)).astype(np.float32)
    inp.k *= rng.uniform(0.05, 20, inp.k.shape[:2] + (1,)).astype(np.float32)
    o2, s2 = run_chunk(inp, fused=fused)
    assert rel_err(o2, o.astype(np.float64)) < 1e-4 and rel_err(s2, s.astype(np.float64)) < 1e-4


def test_split_t_prologue():
    spec = kda_inputs.Spec([8192], 1, 128, 128, "bf16", "softplus", s0_std=0.02, seed=66, gate_dtype="bf16",
                           name="pro-split", **ALL)
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp))


@pytest.mark.parametrize("flags", [dict(), ALL], ids=["bf16_gates_only", "all"])
@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128), (128, 64)])
def test_decode_prologue(Dk, Dv, flags):
    spec = kda_inputs.Spec([1] * 6, 3, Dk, Dv, "bf16", "softplus", s0_std=0.3, seed=67, gate_dtype="bf16",
                           logit_std=2.0 if flags else 1.0, **flags)
    inp = kda_inputs.generate(spec)
    o, s, _ = run_decode(inp)
    o_ref, s_ref = oracle.forward_inputs(inp)
    eo, es = rel_err(o, o_ref.reshape(o.shape)), rel_err(s, s_ref)
    print(f"decode prologue {flags} {Dk}x{Dv}: o err {eo:.3e} S err {es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_decode_prologue_f32_zero_vectors():
    spec = kda_inputs.Spec([1] * 4, 2, 128, 128, "f32", "softplus", s0_std=0.3, seed=68, **ALL)
    inp = kda_inputs.generate(spec)
    inp.q[1] = 0.0
    inp.k[2] = 0.0
    o, s, _ = run_decode(inp)
    o_ref, s_ref = oracle.forward_inputs(inp)
    assert rel_err(o, o_ref.reshape(o.shape)) <= TOL["f32"] and rel_err(s, s_ref) <= TOL["f32"]
    assert not o[1].any()


def test_prologue_rejects_bad_gate_dtype():
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError, match="g must be"):
        kda.chunk_fwd(q, q, q, q.half(), torch.zeros(1, 64, 1, device="cuda"))
