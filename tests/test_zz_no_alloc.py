"""kda_chunk_fwd_noalloc (the entry point for callers that cannot allocate) against kda_chunk_fwd.

Both are called through the C ABI on the same seeded inputs.  The no-allocation call runs the same
kernels over T-windows in the library's fixed per-GPU scratch and carries the state between windows
in fp32, so its results must equal the two-kernel call's bit for bit; they are also held to the
oracle's tolerance.  Two calls in a row share the scratch, the second with a smaller input (and no
s_final, so the carried state lives in the scratch too): whatever the first call left there must not
leak into the second.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_65_amd as kda
import kda_inputs
import oracle
from tests.gpu_util import TOL, device_inputs, rel_err

pytestmark = pytest.mark.gpu


def stream():
    return torch.cuda.current_stream().cuda_stream


def with_workspace(d, B, T, H, Dk, Dv):
    """kda_chunk_fwd, two-kernel path (caller's workspace), through the C ABI."""
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device="cuda")
    sf = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device="cuda")
    nws = kda.chunk_workspace_bytes(B, T, H, Dk, Dv, d["q"].dtype)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    rc = kda.chunk_fwd_raw(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["g"].data_ptr(),
                           d["beta"].data_ptr(), None if d["s0"] is None else d["s0"].data_ptr(), o.data_ptr(),
                           sf.data_ptr(), B, T, H, Dk, Dv, 64, kda.DTYPE[d["q"].dtype], None, ws.data_ptr(), nws,
                           stream())
    assert rc == 0, kda.load_library().kda_last_error()
    return o, sf


def no_alloc(d, B, T, H, Dk, Dv, want_state):
    """kda_chunk_fwd_noalloc through the C ABI (outputs preallocated here, NaN-filled)."""
    o = torch.full((B, T, H, Dv), float("nan"), dtype=torch.float32, device="cuda")
    sf = torch.full((B, H, Dk, Dv), float("nan"), dtype=torch.float32, device="cuda") if want_state else None
    rc = kda.chunk_fwd_noalloc_raw(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["g"].data_ptr(),
                                   d["beta"].data_ptr(), None if d["s0"] is None else d["s0"].data_ptr(),
                                   o.data_ptr(), None if sf is None else sf.data_ptr(), B, T, H, Dk, Dv, 64,
                                   kda.DTYPE[d["q"].dtype], None, stream())
    assert rc == 0, kda.load_library().kda_last_error()
    return o, sf


def test_no_alloc_matches_the_workspace_call_twice():
    # 1) the B=4 H=16 T=8192 d=128 bf16 batch: 64 sequence-heads, several windows of the scratch
    spec = kda_inputs.workload("chunk_b4_h16_t8192_d128_bf16")
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    B, T, H, Dk, Dv = spec.n_seq, spec.lengths[0], spec.H, spec.Dk, spec.Dv
    print(f"no-alloc call 1: B={B} T={T} H={H} d={Dk} bf16", flush=True)
    o_ref, s_ref = with_workspace(d, B, T, H, Dk, Dv)
    o1, s1 = no_alloc(d, B, T, H, Dk, Dv, want_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o_ref) and torch.equal(s1, s_ref)
    ref_o, ref_s = oracle.forward_inputs(inp)
    eo = rel_err(o1.reshape(B * T, H, Dv).cpu().numpy(), ref_o)
    es = rel_err(s1.cpu().numpy(), ref_s)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]

    # 2) a smaller call right after: ragged T, an initial state, no final state (carried in the scratch)
    spec2 = kda_inputs.Spec([200] * 2, 3, 128, 64, "f32", "softplus_bounds", 0.05, s0_std=0.02, seed=91,
                            name="no-alloc-small")
    inp2 = kda_inputs.generate(spec2)
    d2 = device_inputs(inp2, True)
    print("no-alloc call 2: B=2 T=200 H=3 Dk=128 Dv=64 f32, s0 given, no s_final", flush=True)
    o_ref2, _ = with_workspace(d2, 2, 200, 3, 128, 64)
    o2, s2 = no_alloc(d2, 2, 200, 3, 128, 64, want_state=False)
    torch.cuda.synchronize()
    assert s2 is None and torch.equal(o2, o_ref2)
    ref_o2, _ = oracle.forward_inputs(inp2, want_state=False)
    eo2 = rel_err(o2.reshape(400, 3, 64).cpu().numpy(), ref_o2)
    print(f"  o err {eo2:.3e}", flush=True)
    assert eo2 <= TOL["f32"]


def test_no_alloc_edge_cases():
    # T = 0 with a final state: s0 passes through (no scratch used)
    s0 = torch.randn((2, 2, 128, 128), device="cuda")
    sf = torch.full_like(s0, float("nan"))
    rc = kda.chunk_fwd_noalloc_raw(None, None, None, None, None, s0.data_ptr(), None, sf.data_ptr(), 2, 0, 2, 128,
                                   128, 64, kda.DTYPE[torch.bfloat16], None, stream())
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(sf, s0)
    # one token, the torch front end
    spec = kda_inputs.Spec([1], 2, 64, 64, "bf16", "softplus", s0_std=0.02, seed=92, name="no-alloc-1")
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    o, s = kda.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                 s_final=torch.empty((1, 2, 64, 64), device="cuda"))
    o_ref, s_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
