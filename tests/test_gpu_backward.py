"""GPU parity of the backward pass against the oracle's fp64 reverse mode.

Loss L = <d_o, o> + <d_sfinal, S_T> with seeded random d_o, d_sfinal; every gradient (dq, dk, dv,
dg, dbeta, ds0) is compared element by element: max|gpu - oracle| <= tol * RMS(oracle) per tensor.
The kernels accumulate in fp32 and run their products in fp32 or as three-pass split-bf16 products
for both input types, so one tolerance serves both.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_65_amd as kda
import kda_inputs
import oracle
from tests.gpu_util import device_inputs, rel_err, to_dev

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-3
NAMES = ["dq", "dk", "dv", "dg", "dbeta", "ds0"]


def cotangents(spec, seed):
    rng = np.random.default_rng(seed)
    d_o = rng.standard_normal((spec.total, spec.H, spec.Dv)).astype(np.float32)
    d_sf = (0.1 * rng.standard_normal((spec.n_seq, spec.H, spec.Dk, spec.Dv))).astype(np.float32)
    return d_o, d_sf


def run_bwd(inp, d_o, d_sf, batched=True, with_dsf=True, workspace=None):
    sp = inp.spec
    d = device_inputs(inp, batched)
    dsf = to_dev(d_sf) if with_dsf else None
    if batched:
        B, T = sp.n_seq, sp.lengths[0]
        out = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], to_dev(d_o, (B, T, sp.H, sp.Dv)), d["s0"],
                            dsf, workspace=workspace)
    else:
        out = kda.varlen_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], to_dev(d_o), d["s0"], dsf,
                             workspace=workspace)
    torch.cuda.synchronize()
    res = {}
    for name, t in zip(NAMES, out):
        a = t.cpu().numpy()
        if name in ("dq", "dk", "dg"):
            a = a.reshape(sp.total, sp.H, sp.Dk)
        elif name == "dv":
            a = a.reshape(sp.total, sp.H, sp.Dv)
        elif name == "dbeta":
            a = a.reshape(sp.total, sp.H)
        res[name] = a
    return res


def reference(inp, d_o, d_sf, with_dsf=True):
    return oracle.backward(inp.as_f32("q"), inp.as_f32("k"), inp.as_f32("v"), inp.as_f32("g"), inp.as_f32("beta"),
                           inp.cu_seqlens, d_o, s0=inp.s0, d_sfinal=d_sf if with_dsf else None)


def check(inp, gpu, ref, tol=BWD_TOL):
    errs = {n: rel_err(gpu[n], ref[n]) for n in NAMES}
    print(f"[bwd {inp.spec.name or inp.spec.lengths[:4]}] " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return errs


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_ragged_lengths(T, dtype):
    spec = kda_inputs.Spec([T] * 2, 2, 128, 128, dtype, "softplus_bounds", 0.05, s0_std=0.02, seed=70 + T,
                           name=f"bwd-T{T}-{dtype}")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, T)
    check(inp, run_bwd(inp, d_o, d_sf), reference(inp, d_o, d_sf))


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_backward_head_dims(Dk, Dv):
    spec = kda_inputs.Spec([150] * 2, 2, Dk, Dv, "f32", "softplus", s0_std=0.1, seed=80, name=f"bwd-{Dk}x{Dv}")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 1)
    check(inp, run_bwd(inp, d_o, d_sf), reference(inp, d_o, d_sf))


def test_backward_long_sequences():
    spec = kda_inputs.Spec([2048] * 2, 4, 128, 128, "bf16", "softplus_bounds", 0.05, s0_std=0.02, seed=81,
                           name="bwd-2048")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 2)
    check(inp, run_bwd(inp, d_o, d_sf), reference(inp, d_o, d_sf))


def test_backward_workload_chunk_b4_h16_t8192_d128_bf16():
    """The benchmarked backward call: B=4 H=16 T=8192 d=128 bf16 (bound-forced gates), no final-state
    gradient, every gradient of the whole batch against the oracle's fp64 reverse mode."""
    spec = kda_inputs.workload("chunk_b4_h16_t8192_d128_bf16")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 5)
    check(inp, run_bwd(inp, d_o, d_sf, with_dsf=False), reference(inp, d_o, d_sf, with_dsf=False))


def test_backward_long_memory_gate():
    spec = kda_inputs.Spec([1500], 2, 128, 128, "bf16", "longmem", seed=82, name="bwd-longmem")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 3)
    check(inp, run_bwd(inp, d_o, d_sf), reference(inp, d_o, d_sf))


def test_backward_varlen_with_empty():
    spec = kda_inputs.Spec([0, 1, 64, 65, 130, 0, 7], 3, 128, 128, "bf16", "softplus", s0_std=0.02, seed=83,
                           packed=True, name="bwd-varlen")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 4)
    gpu = run_bwd(inp, d_o, d_sf, batched=False)
    check(inp, gpu, reference(inp, d_o, d_sf))
    # empty sequences pass the final-state gradient straight to the initial state
    assert np.array_equal(gpu["ds0"][0], d_sf[0]) and np.array_equal(gpu["ds0"][5], d_sf[5])


def test_backward_without_final_state_gradient():
    spec = kda_inputs.Spec([130] * 2, 2, 128, 128, "bf16", "softplus", s0_std=0.02, seed=84, name="bwd-nodsf")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 5)
    check(inp, run_bwd(inp, d_o, d_sf, with_dsf=False), reference(inp, d_o, d_sf, with_dsf=False))


def test_backward_clamp_mask():
    """g outside [-5, 0] gets exactly zero gradient."""
    spec = kda_inputs.Spec([100] * 2, 2, 128, 128, "f32", "softplus", s0_std=0.1, seed=85, name="bwd-clamp")
    inp = kda_inputs.generate(spec)
    rng = np.random.default_rng(0)
    inp.g[:] = rng.uniform(-7.0, 1.5, inp.g.shape).astype(np.float32)
    d_o, d_sf = cotangents(spec, 6)
    gpu = run_bwd(inp, d_o, d_sf)
    check(inp, gpu, reference(inp, d_o, d_sf))
    outside = (inp.g < -5) | (inp.g > 0)
    assert outside.any() and np.all(gpu["dg"][outside] == 0.0)


def test_backward_infinite_gates():
    """log alpha = -inf / +inf act as the bounds in every gradient and get a zero gradient themselves."""
    spec = kda_inputs.Spec([100] * 2, 2, 128, 128, "bf16", "softplus", s0_std=0.1, seed=86, name="bwd-inf")
    inp = kda_inputs.generate(spec)
    sel = np.random.default_rng(1).integers(0, 6, size=inp.g.shape)
    inp.g[sel == 0] = -np.inf
    inp.g[sel == 1] = np.inf
    d_o, d_sf = cotangents(spec, 7)
    gpu = run_bwd(inp, d_o, d_sf)
    for n in NAMES:
        assert np.isfinite(gpu[n]).all(), n
    check(inp, gpu, reference(inp, d_o, d_sf))
    assert np.all(gpu["dg"][sel <= 1] == 0.0)


def test_backward_workspace_reused_and_dirty():
    spec = kda_inputs.Spec([200] * 2, 2, 128, 128, "bf16", "softplus", s0_std=0.02, seed=86, name="bwd-ws")
    inp = kda_inputs.generate(spec)
    d_o, d_sf = cotangents(spec, 7)
    need = kda.chunk_bwd_workspace_bytes(2, 200, 2, 128, 128)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    a = run_bwd(inp, d_o, d_sf, workspace=ws)
    b = run_bwd(inp, d_o, d_sf, workspace=ws)
    check(inp, a, reference(inp, d_o, d_sf))
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_autograd_function_matches_direct_call():
    spec = kda_inputs.Spec([96] * 2, 2, 128, 128, "f32", "softplus", s0_std=0.1, seed=87)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ["q", "k", "v", "g", "beta", "s0"]}
    o, sf = kda.ChunkKDA.apply(*(leaves[n] for n in ["q", "k", "v", "g", "beta", "s0"]))
    d_o, d_sf = cotangents(spec, 8)
    d_o_t = to_dev(d_o, o.shape)
    d_sf_t = to_dev(d_sf)
    torch.autograd.backward([o, sf], [d_o_t, d_sf_t])
    direct = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o_t, d["s0"], d_sf_t)
    torch.cuda.synchronize()
    for n, t in zip(["q", "k", "v", "g", "beta", "s0"], direct):
        assert torch.equal(leaves[n].grad, t), n


def test_backward_rejects_missing_workspace():
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(1, 64, 1, 128, device="cuda")
    dq = torch.empty_like(z)
    b = torch.zeros(1, 64, 1, device="cuda")
    rc = kda.chunk_bwd_raw(q.data_ptr(), q.data_ptr(), q.data_ptr(), z.data_ptr(), b.data_ptr(), None, z.data_ptr(),
                           None, dq.data_ptr(), dq.data_ptr(), dq.data_ptr(), dq.data_ptr(), b.data_ptr(), None,
                           1, 64, 1, 128, 128, 64, 1, None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 1 and "workspace" in kda.load_library().kda_last_error().decode()
