"""GPU parity: the HIP path against the fp64 CPU oracle on the same seeded inputs.

Metric: max|gpu - oracle| / RMS(oracle) over the whole output (o) and final
state, <= 2e-2 for bf16 inputs and <= 1e-4 for fp32 inputs.  Full-size
workloads compare a sample of state columns (columns of the state evolve
independently, so the oracle computes them exactly on their own).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_65_amd as kda
import kda_inputs
import oracle
from tests.gpu_util import TOL, device_inputs, rel_err, to_dev

pytestmark = pytest.mark.gpu

# both implementations of the prefill entry points: the two-kernel path (with a workspace)
# and the single fused kernel (workspace NULL)
PATHS = pytest.mark.parametrize("fused", [False, True], ids=["two_pass", "fused"])


def prologue_flags(spec):
    """The input prologue that the spec's raw input forms call for."""
    return dict(g_logit=spec.g_logit, beta_logit=spec.beta_logit, qk_l2norm=spec.qk_l2norm)


def run_chunk(inp, batched=True, fused=False, workspace=None):
    d = device_inputs(inp, batched)
    fl = prologue_flags(inp.spec)
    if batched:
        o, sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], fused=fused, workspace=workspace,
                              **fl)
    else:
        o, sf = kda.varlen_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["s0"], fused=fused,
                               workspace=workspace, **fl)
    torch.cuda.synchronize()
    sp = inp.spec
    return o.reshape(sp.total, sp.H, sp.Dv).cpu().numpy(), sf.cpu().numpy()


_ORACLE_CACHE = {}


def reference(inp, cols=None):
    """Oracle outputs; those of the named workloads are kept for the test of the other path."""
    key = (inp.spec.name, tuple(cols) if cols is not None else None)
    if inp.spec.name in kda_inputs.WORKLOADS:
        if key not in _ORACLE_CACHE:
            _ORACLE_CACHE[key] = oracle.forward_inputs(inp, cols=cols)
        return _ORACLE_CACHE[key]
    return oracle.forward_inputs(inp, cols=cols)


def check(inp, o_gpu, s_gpu, cols=None, tol=None):
    tol = tol or TOL[inp.spec.dtype]
    o_ref, s_ref = reference(inp, cols=cols)
    if cols is not None:
        o_gpu, s_gpu = o_gpu[..., cols], s_gpu[..., cols]
    eo, es = rel_err(o_gpu, o_ref), rel_err(s_gpu, s_ref)
    print(f"[{inp.spec.name or inp.spec.lengths[:4]}] o err {eo:.3e}  S err {es:.3e}  (tol {tol})", flush=True)
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


# ----------------------------------------------------------------- the five named workloads

@PATHS
def test_workload_chunk_b1_h1_t256_d64_f32(fused):
    inp = kda_inputs.generate(kda_inputs.workload("chunk_b1_h1_t256_d64_f32"))
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
def test_workload_chunk_b4_h16_t8192_d128_bf16(fused):
    inp = kda_inputs.generate(kda_inputs.workload("chunk_b4_h16_t8192_d128_bf16"))
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
def test_workload_varlen_n32_h16_d128_bf16(fused):
    inp = kda_inputs.generate(kda_inputs.workload("varlen_n32_h16_d128_bf16"))
    cols = [0, 17, 31, 32, 63, 64, 100, 127]
    check(inp, *run_chunk(inp, batched=False, fused=fused), cols=cols)


# ----------------------------------------------------------------- edge cases and shapes

@PATHS
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_lengths(T, dtype, fused):
    spec = kda_inputs.Spec([T] * 2, 3, 128, 128, dtype, "softplus_bounds", 0.05, s0_std=0.02, seed=11 + T,
                           name=f"T{T}-{dtype}")
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dims(Dk, Dv, dtype, fused):
    spec = kda_inputs.Spec([150] * 2, 2, Dk, Dv, dtype, "softplus", s0_std=0.02, seed=5, name=f"{Dk}x{Dv}-{dtype}")
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, fused=fused))


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128)])
@pytest.mark.parametrize("packed", [False, True], ids=["batched", "packed"])
def test_more_chains_than_compute_units(Dk, Dv, packed):
    """Chain grids larger than the CU count (576 and 640 workgroups) run in several rounds."""
    lengths = [130] * 9 if not packed else [1, 64, 65, 200, 0, 127, 129, 90, 33, 256]
    spec = kda_inputs.Spec(lengths, 16, Dk, Dv, "bf16", "softplus", s0_std=0.02, seed=21, packed=packed,
                           name=f"many-chains-{Dk}x{Dv}-{'packed' if packed else 'batched'}")
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, batched=not packed))


def beyond_bounds(inp, seed):
    """Set a fifth of the gates each to -inf, -1e4, +3 and +inf (all outside [-5, 0])."""
    sel = np.random.default_rng(seed).integers(0, 5, size=inp.g.shape)
    for i, val in enumerate([-np.inf, -1e4, 3.0, np.inf]):
        inp.g[sel == i] = val
    return inp


@PATHS
def test_gates_beyond_the_clamp_bounds(fused):
    """log alpha outside [-5, 0], infinities included, acts as the nearest bound."""
    spec = kda_inputs.Spec([150] * 2, 3, 128, 128, "bf16", "softplus", s0_std=0.02, seed=41, name="gates-beyond")
    inp = beyond_bounds(kda_inputs.generate(spec), 41)
    o, s = run_chunk(inp, fused=fused)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    check(inp, o, s)


def scale_bf16(bits, factor):
    """bf16 bit patterns times a power of two (exact)."""
    return kda_inputs.f32_to_bf16_bits(kda_inputs.bf16_bits_to_f32(bits) * np.float32(factor))


def check_rows(o_gpu, o_ref, rows, tol, what):
    e = rel_err(o_gpu[rows], o_ref[rows])
    print(f"  {what}: o err {e:.3e}", flush=True)
    assert e <= tol, (what, e)


@PATHS
def test_values_beyond_half_precision_range(fused):
    """Values up to about 2^18 and an initial state up to about 2^14 (half precision ends at 65504):
    the bf16 bar holds on the output and the final state."""
    spec = kda_inputs.Spec([640] * 2, 2, 128, 128, "bf16", "softplus_bounds", 0.05, s0_std=0.02, seed=43,
                           name="wide-range")
    inp = kda_inputs.generate(spec)
    inp.v = scale_bf16(inp.v, 2.0 ** 16)
    inp.s0 = (inp.s0 * np.float32(2.0 ** 16)).astype(np.float32)
    o, s = run_chunk(inp, fused=fused)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    check(inp, o, s)


@PATHS
def test_value_spike(fused):
    """One chunk of values 2^20 larger than the rest in the middle of each sequence.  Everything but the
    chunk after it keeps the bf16 bar: the rows before the spike, the rows from the second chunk after
    it on (each against its own scale), the whole output and the final state.  The chunk right after
    the spike holds the spike's decay over six orders of magnitude within one chunk; it is only
    required to be finite."""
    spec = kda_inputs.Spec([640] * 2, 2, 128, 128, "bf16", "softplus_bounds", 0.05, s0_std=0.02, seed=43,
                           name="value-spike")
    inp = kda_inputs.generate(spec)
    inp.v = scale_bf16(inp.v, 2.0 ** 12)
    v = inp.v.reshape(2, 640, 2, 128)
    v[:, 320:384] = scale_bf16(v[:, 320:384], 2.0 ** 20)
    o, s = run_chunk(inp, fused=fused)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    tol = TOL["bf16"]
    check(inp, o, s)
    o_ref, _ = reference(inp)
    ob, rb = o.reshape(2, 640, 2, 128), o_ref.reshape(2, 640, 2, 128)
    check_rows(ob, rb, np.s_[:, :320], tol, "before the spike")
    for c in range(7, 10):
        check_rows(ob, rb, np.s_[:, 64 * c:64 * (c + 1)], tol, f"chunk {c}")


@PATHS
def test_state_growing_past_value_range(fused):
    """Keys of 2^-5 on two coordinates with beta = 1, no decay and v = 60 everywhere drive those state
    rows toward 60 / 2^-5 = 1920 (thirty times the largest value), so the state alone sets the
    working range part way through the sequence."""
    T, H, D = 4096, 2, 128
    spec = kda_inputs.Spec([T], H, D, D, "bf16", "softplus", seed=44, name="state-growth")
    inp = kda_inputs.generate(spec)
    k = np.zeros((T, H, D), np.float32)
    t = np.arange(T)
    k[t, :, (t % 2) * 37] = 2.0 ** -5
    inp.k = kda_inputs.f32_to_bf16_bits(k)
    inp.v = kda_inputs.f32_to_bf16_bits(np.full((T, H, D), 60.0, np.float32))
    inp.g[:] = 0.0
    inp.beta[:] = 1.0
    o, s = run_chunk(inp, fused=fused)
    _, s_ref = reference(inp)
    assert np.abs(s_ref).max() > 1024.0  # the state outgrows 2^10 while |v| < 2^6
    check(inp, o, s)


@PATHS
def test_long_memory_gate(fused):
    spec = kda_inputs.Spec([2048], 4, 128, 128, "bf16", "longmem", seed=4, name="longmem-2048")
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp, fused=fused))


@PATHS
def test_varlen_ragged_with_empty(fused):
    spec = kda_inputs.Spec([0, 1, 64, 65, 130, 0, 7], 3, 128, 128, "bf16", "softplus", s0_std=0.02, seed=9,
                           packed=True, name="varlen-edge")
    inp = kda_inputs.generate(spec)
    o, s = run_chunk(inp, batched=False, fused=fused)
    check(inp, o, s)
    # empty sequences pass their initial state through unchanged
    assert np.array_equal(s[0], inp.s0[0]) and np.array_equal(s[5], inp.s0[5])


@PATHS
def test_zero_length_returns_initial_state(fused):
    spec = kda_inputs.Spec([0, 0], 2, 128, 64, "bf16", s0_std=0.5, seed=3)
    inp = kda_inputs.generate(spec)
    s0 = to_dev(inp.s0)
    q = torch.empty(2, 0, 2, 128, dtype=torch.bfloat16, device=s0.device)
    v = torch.empty(2, 0, 2, 64, dtype=torch.bfloat16, device=s0.device)
    o, sf = kda.chunk_fwd(q, q, v, q.float(), torch.empty(2, 0, 2, device=s0.device), s0, fused=fused)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(sf, s0)
    _, sz = kda.chunk_fwd(q, q, v, q.float(), torch.empty(2, 0, 2, device=s0.device), None, fused=fused)
    torch.cuda.synchronize()
    assert not sz.any()


# ----------------------------------------------------------------- invariants on the GPU

@PATHS
def test_identity_gate_keeps_state(fused):
    """alpha = 1, beta = 0: S_T = S0 and o_t = S0^T q_t."""
    spec = kda_inputs.Spec([130] * 2, 2, 128, 128, "f32", "softplus", s0_std=0.3, seed=21)
    inp = kda_inputs.generate(spec)
    inp.g[:] = 0.0
    inp.beta[:] = 0.0
    o, s = run_chunk(inp, fused=fused)
    np.testing.assert_allclose(s, inp.s0, rtol=0, atol=1e-6)
    check(inp, o, s)


@PATHS
def test_zero_in_zero_out(fused):
    spec = kda_inputs.Spec([100] * 2, 2, 128, 128, "bf16", "softplus", seed=22)
    inp = kda_inputs.generate(spec)
    inp.q[:] = 0
    inp.k[:] = 0
    inp.v[:] = 0
    o, s = run_chunk(inp, fused=fused)
    assert not o.any() and not s.any()


@PATHS
def test_unit_key_full_write(fused):
    """beta = 1 with unit keys (coordinate axes): k_t^T S_t = v_t; with q = k, o_t = v_t."""
    T, H, D = 96, 2, 128
    spec = kda_inputs.Spec([T], H, D, D, "f32", "softplus", seed=23)
    inp = kda_inputs.generate(spec)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, D, (T, H))
    inp.k[:] = 0
    inp.k[np.arange(T)[:, None], np.arange(H)[None, :], idx] = 1.0
    inp.q[:] = inp.k
    inp.beta[:] = 1.0
    o, s = run_chunk(inp, fused=fused)
    np.testing.assert_allclose(o, inp.v, rtol=0, atol=1e-4)


@PATHS
def test_split_resume_matches_unbroken(fused):
    spec = kda_inputs.Spec([256], 2, 128, 128, "bf16", "softplus_bounds", 0.05, s0_std=0.02, seed=24)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    o, sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], fused=fused)
    T1 = 100
    sl = lambda x, a, b: x[:, a:b].contiguous()
    oa, sa = kda.chunk_fwd(*(sl(d[n], 0, T1) for n in "q k v g beta".split()), d["s0"], fused=fused)
    ob, sb = kda.chunk_fwd(*(sl(d[n], T1, 256) for n in "q k v g beta".split()), sa, fused=fused)
    torch.cuda.synchronize()
    # the split moves every chunk boundary after T1, so the two runs round differently: both are held
    # to the oracle's bar, and to each other within twice the error either shows on these gates
    ref = o.cpu().numpy()
    split = torch.cat([oa, ob], 1).cpu().numpy()
    o_ref, s_ref = reference(inp)
    for oo, ss in ((split, sb), (ref, sf)):
        assert rel_err(oo.reshape(256, 2, 128), o_ref) <= TOL["bf16"]
        assert rel_err(ss.cpu().numpy(), s_ref) <= TOL["bf16"]
    assert rel_err(split, ref) < 1e-2 and rel_err(sb.cpu().numpy(), sf.cpu().numpy()) < 1e-2


@PATHS
def test_varlen_equals_batched(fused):
    spec = kda_inputs.Spec([192] * 3, 2, 128, 128, "bf16", "softplus", s0_std=0.02, seed=25)
    inp = kda_inputs.generate(spec)
    ob, sb = run_chunk(inp, batched=True, fused=fused)
    ov, sv = run_chunk(inp, batched=False, fused=fused)
    assert np.array_equal(ob, ov) and np.array_equal(sb, sv)


@pytest.mark.parametrize("T,H,Dk,Dv,dtype,with_s0", [
    (8192, 1, 128, 128, "bf16", True),     # 2 segments
    (16421, 2, 128, 128, "bf16", True),    # 4 uneven segments, ragged last chunk
    (12800, 1, 128, 64, "bf16", False),    # 3 segments, Dv = 64
    (8192, 1, 64, 64, "f32", True),        # fp32, Dk = 64
])
def test_split_t_segments(T, H, Dk, Dv, dtype, with_s0):
    """Few heads, long sequence: the chunk range is cut into segments (zero-start runs and
    transitions, fold, output pass); results match the token recurrence."""
    spec = kda_inputs.Spec([T], H, Dk, Dv, dtype, "softplus_bounds", 0.05, s0_std=0.02 if with_s0 else None,
                           seed=50 + T % 97, name=f"split-T{T}-H{H}-{Dk}x{Dv}-{dtype}")
    inp = kda_inputs.generate(spec)
    check(inp, *run_chunk(inp))


def test_long_split_call_in_windows(monkeypatch):
    """A split call whose records exceed the window budget runs as T-windows, each a split call of
    its own, with the state carried between them: four windows of 256 chunks, four segments each."""
    monkeypatch.setenv("KDA_SPLIT_WINDOW_BYTES", str(40 << 20))
    spec = kda_inputs.Spec([65536], 2, 128, 128, "bf16", "softplus_bounds", 0.05, s0_std=0.02, seed=45,
                           name="split-windows")
    inp = kda_inputs.generate(spec)
    B, T, H = 1, 65536, 2
    assert kda.chunk_workspace_bytes(B, T, H, 128, 128) < B * (T // 64) * H * 74240  # windowed
    check(inp, *run_chunk(inp))


def test_two_pass_with_caller_workspace_reused_and_dirty():
    """The workspace needs no initial contents and one buffer serves calls of different sizes."""
    big = kda_inputs.generate(kda_inputs.Spec([300] * 2, 3, 128, 128, "bf16", "softplus_bounds", 0.05,
                                              s0_std=0.02, seed=31, name="ws-big"))
    small = kda_inputs.generate(kda_inputs.Spec([70, 0, 129], 3, 128, 128, "bf16", "softplus", s0_std=0.02,
                                                seed=32, packed=True, name="ws-small"))
    need = kda.chunk_workspace_bytes(2, 300, 3, 128, 128)
    assert kda.varlen_workspace_bytes(3, 199, 3, 128, 128) <= need
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    check(big, *run_chunk(big, workspace=ws))
    check(small, *run_chunk(small, batched=False, workspace=ws))
    ref_o, ref_s = run_chunk(big)
    o2, s2 = run_chunk(big, workspace=ws)
    assert np.array_equal(o2, ref_o) and np.array_equal(s2, ref_s)


def test_two_pass_rejects_small_workspace():
    inp = kda_inputs.generate(kda_inputs.Spec([128], 1, 128, 128, "bf16", seed=33))
    ws = torch.empty(kda.chunk_workspace_bytes(1, 128, 1, 128, 128) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kda.KDAError, match="workspace"):
        run_chunk(inp, workspace=ws)


@PATHS
def test_bitwise_repeatable(fused):
    spec = kda_inputs.Spec([300] * 2, 4, 128, 128, "bf16", "softplus_bounds", 0.05, seed=26)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    o1, s1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], fused=fused)
    o2, s2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], fused=fused)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@PATHS
def test_s_final_may_alias_s0(fused):
    spec = kda_inputs.Spec([130] * 2, 2, 128, 128, "bf16", "softplus", s0_std=0.02, seed=27)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    o, sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], fused=fused)
    st = d["s0"].clone()
    o2 = torch.empty_like(o)
    nws = 0 if fused else kda.chunk_workspace_bytes(2, 130, 2, 128, 128)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    rc = kda.chunk_fwd_raw(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["g"].data_ptr(),
                           d["beta"].data_ptr(), st.data_ptr(), o2.data_ptr(), st.data_ptr(), 2, 130, 2, 128, 128,
                           64, kda.DTYPE[torch.bfloat16], None, None if fused else ws.data_ptr(), nws,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(st, sf) and torch.equal(o2, o)


def test_s_final_may_alias_s0_split_t():
    """One long sequence with one head runs as a split-T segment scan (P = 2 segments): s0 is read
    by the segment fold, s_final written by the last segment's workgroups; aliasing the two is safe."""
    spec = kda_inputs.Spec([8192], 1, 128, 128, "bf16", "softplus", s0_std=0.02, seed=28)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, True)
    o, sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    st = d["s0"].clone()
    o2 = torch.empty_like(o)
    nws = kda.chunk_workspace_bytes(1, 8192, 1, 128, 128)
    assert nws > 128 * kda.chunk_workspace_bytes(1, 64, 1, 128, 128)  # the segment states are part of it
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    rc = kda.chunk_fwd_raw(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["g"].data_ptr(),
                           d["beta"].data_ptr(), st.data_ptr(), o2.data_ptr(), st.data_ptr(), 1, 8192, 1, 128, 128,
                           64, kda.DTYPE[torch.bfloat16], None, ws.data_ptr(), nws,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(st, sf) and torch.equal(o2, o)
    check(inp, o.reshape(8192, 1, 128).cpu().numpy(), sf.cpu().numpy())


def test_varlen_without_tokens_takes_the_queried_workspace():
    """total = 0: the size query returns 0, and a call given that size passes s0 to s_final."""
    N, H = 3, 2
    assert kda.varlen_workspace_bytes(N, 0, H, 128, 128) == 0
    s0 = torch.randn((N, H, 128, 128), device="cuda")
    sf = torch.full_like(s0, float("nan"))
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    rc = kda.varlen_fwd_raw(None, None, None, None, None, cu.data_ptr(), N, 0, s0.data_ptr(), None, sf.data_ptr(),
                            H, 128, 128, 64, kda.DTYPE[torch.bfloat16], None, ws.data_ptr(), 0,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0, kda.load_library().kda_last_error()
    assert torch.equal(sf, s0)


def test_workload_prefill_b1_h8_t1m_d128_bf16():
    """Million-token prefill (long-memory gate): final state and outputs on sampled state
    columns, each computed exactly by the oracle on its own (columns are independent)."""
    spec = kda_inputs.workload("prefill_b1_h8_t1m_d128_bf16")
    inp = kda_inputs.generate(spec)
    o, s = run_chunk(inp)
    cols = [0, 45, 70, 127]  # one column in each 32-column chain slice
    eo, es = check(inp, o, s, cols=cols)
    # the state after a million tokens stays bounded (the update is a contraction plus a write)
    assert np.isfinite(s).all() and np.abs(s).max() < 1e3
