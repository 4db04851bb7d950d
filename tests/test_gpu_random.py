"""Seeded random parity sweep: the forward and backward entry points on shapes drawn at random
(batched and packed layouts, ragged and empty sequences, head dims 64/128 in every pairing, bf16 and
fp32, the three gate regimes, with and without an initial state, the raw-input prologue, both
prefill paths) against the fp64 oracle, each case to the same tolerance as the fixed tests.
"""
import random

import numpy as np
import pytest
import torch

import gated_delta_rule_65_amd as kda
import kda_inputs
import oracle
from tests.gpu_util import TOL, device_inputs, rel_err
from tests.test_gpu_backward import BWD_TOL, NAMES, cotangents, reference as bwd_reference, run_bwd

pytestmark = pytest.mark.gpu

N_FWD, N_BWD = 48, 16


def fwd_case(i):
    rng = random.Random(1000 + i)
    packed = rng.random() < 0.4
    H = rng.choice([1, 2, 3, 5])
    Dk, Dv = rng.choice([(64, 64), (128, 128), (64, 128), (128, 64)])
    dtype = rng.choice(["bf16", "bf16", "f32"])
    s0 = rng.choice([None, 0.02])
    if packed:
        lengths = [rng.choice([0, 1, 63, 64, 65, rng.randint(1, 600)]) for _ in range(rng.randint(1, 6))]
    else:
        lengths = [rng.choice([1, 64, 65, 127, 128, rng.randint(1, 700)])] * rng.randint(1, 3)
    raw = rng.random() < 0.25
    gate = "softplus" if raw else rng.choice(["softplus", "softplus_bounds", "longmem"])
    spec = kda_inputs.Spec(lengths, H, Dk, Dv, dtype, gate, 0.05, s0, seed=2000 + i, packed=packed, g_logit=raw,
                           beta_logit=raw, qk_l2norm=raw and rng.random() < 0.5,
                           gate_dtype=rng.choice(["f32", "bf16"]) if raw else "f32")
    return spec, rng.random() < 0.3


@pytest.mark.parametrize("i", range(N_FWD))
def test_random_forward(i):
    spec, fused = fwd_case(i)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, not spec.packed)
    fl = dict(g_logit=spec.g_logit, beta_logit=spec.beta_logit, qk_l2norm=spec.qk_l2norm)
    if spec.packed:
        o, sf = kda.varlen_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["s0"], fused=fused, **fl)
    else:
        o, sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], fused=fused, **fl)
    torch.cuda.synchronize()
    o = o.reshape(spec.total, spec.H, spec.Dv).cpu().numpy()
    sf = sf.cpu().numpy()
    o_ref, s_ref = oracle.forward_inputs(inp)
    eo = rel_err(o, o_ref) if o.size else 0.0
    es = rel_err(sf, s_ref)
    print(f"[random fwd {i}] {spec.lengths[:6]} H={spec.H} D={spec.Dk}/{spec.Dv} {spec.dtype} {spec.gate} "
          f"fused={fused}: o {eo:.2e} S {es:.2e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(sf).all()
    assert eo <= TOL[spec.dtype] and es <= TOL[spec.dtype], (eo, es)


@pytest.mark.parametrize("i", range(N_BWD))
def test_random_backward(i):
    rng = random.Random(3000 + i)
    packed = rng.random() < 0.4
    H = rng.choice([1, 2, 3])
    Dk, Dv = rng.choice([(64, 64), (128, 128), (64, 128), (128, 64)])
    if packed:
        lengths = [rng.choice([0, 1, 63, 64, 65, rng.randint(1, 400)]) for _ in range(rng.randint(1, 5))]
    else:
        lengths = [rng.choice([1, 64, 65, 128, rng.randint(1, 400)])] * rng.randint(1, 3)
    spec = kda_inputs.Spec(lengths, H, Dk, Dv, rng.choice(["bf16", "f32"]),
                           rng.choice(["softplus", "softplus_bounds", "longmem"]), 0.05, rng.choice([None, 0.02]),
                           seed=4000 + i, packed=packed)
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 5000 + i)
    with_dsf = rng.random() < 0.7
    gpu = run_bwd(inp, d_o, d_sf, batched=not packed, with_dsf=with_dsf)
    ref = bwd_reference(inp, d_o, d_sf, with_dsf=with_dsf)
    errs = {n: (rel_err(gpu[n], ref[n]) if ref[n].size else 0.0) for n in NAMES}
    print(f"[random bwd {i}] {lengths[:5]} H={H} D={Dk}/{Dv} {spec.dtype} {spec.gate}: "
          + " ".join(f"{n} {e:.1e}" for n, e in errs.items()), flush=True)
    for n in NAMES:
        assert np.isfinite(gpu[n]).all(), n
        assert errs[n] <= BWD_TOL, (n, errs[n])
