"""The C ABI: symbols, host-side validation (no GPU needed: every case below is
rejected before any HIP call)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_65_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

FAKE = 1 << 20  # 16-byte aligned stand-in address; never dereferenced because validation fails first


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(kda_[a-z_0-9]+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions([HEADER])
    for n in ["kda_chunk_fwd", "kda_varlen_fwd", "kda_decode_step", "kda_last_error", "kda_version",
              "kda_chunk_workspace_bytes", "kda_varlen_workspace_bytes", "kda_chunk_fwd_noalloc"]:
        assert n in names
    assert {"kda_calib_copy", "kda_calib_mfma"} <= set(declared_functions())


@pytest.mark.parametrize("args", [(None, FAKE, 1 << 20), (FAKE, None, 1 << 20), (FAKE + 4, FAKE, 1 << 20),
                                  (FAKE, FAKE + 8, 1 << 20), (FAKE, FAKE, 100)])
def test_calib_copy_validation(args):
    assert kda.calib_copy_raw(*args, None) == 2


@pytest.mark.parametrize("args", [(None, 1, 1, 0), (FAKE, 0, 1, 0), (FAKE, 1, 0, 0), (FAKE, 1, 1, 2)])
def test_calib_mfma_validation(args):
    assert kda.calib_mfma_raw(*args, None) == 2


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kda.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_version():
    assert kda.load_library().kda_version().decode().startswith("kda-gfx950")


def last_error():
    return kda.load_library().kda_last_error().decode()


def chunk(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, o=FAKE, s_final=None, B=1, T=64, H=1, Dk=128,
             Dv=128, chunk=64, dtype=1, prologue=None, workspace=None, workspace_bytes=0, stream=None)
    a.update(kw)
    return kda.chunk_fwd_raw(*a.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Dk=96), 2, "Dk"), (dict(Dv=32), 2, "Dv"), (dict(H=0), 2, "H"), (dict(chunk=32), 2, "chunk"),
    (dict(T=-1), 2, "T"), (dict(B=-2), 2, "B"), (dict(dtype=7), 3, "dtype"),
    (dict(q=None), 1, "q"), (dict(k=None), 1, "k"), (dict(v=None), 1, "v"), (dict(g=None), 1, "g"),
    (dict(beta=None), 1, "beta"), (dict(o=None), 1, "o"),
    (dict(q=FAKE + 2), 4, "q"), (dict(v=FAKE + 8), 4, "v"), (dict(s0=FAKE + 4), 4, "s0"),
    (dict(s_final=FAKE + 12), 4, "s_final"), (dict(workspace=FAKE + 8, workspace_bytes=1 << 30), 4, "workspace"),
    (dict(workspace=FAKE, workspace_bytes=74239), 2, "workspace"),
])
def test_chunk_validation(kw, status, msg):
    assert chunk(**kw) == status
    assert msg in last_error()


def test_chunk_nothing_to_do_returns_ok():
    # no tokens and no final state requested: nothing is launched
    assert chunk(q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == 0
    assert chunk(B=0) == 0
    assert last_error() == ""


def chunk_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, o=FAKE, s_final=None, B=1, T=64, H=1, Dk=128,
             Dv=128, chunk=64, dtype=1, prologue=None, stream=None)
    a.update(kw)
    return kda.chunk_fwd_noalloc_raw(*a.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Dk=96), 2, "Dk"), (dict(chunk=32), 2, "chunk"), (dict(T=-1), 2, "T"), (dict(dtype=7), 3, "dtype"),
    (dict(q=None), 1, "q"), (dict(o=None), 1, "o"), (dict(s_final=FAKE + 4), 4, "s_final"),
    # one 64-token window of 1808 sequence-heads needs more than the fixed 128 MiB scratch (74240 B each)
    (dict(B=1808, s_final=FAKE), 2, "scratch"),
    # without s_final the carried state (64 KiB per sequence-head) lives in the scratch too
    (dict(B=961), 2, "scratch"),
])
def test_chunk_noalloc_validation(kw, status, msg):
    assert chunk_noalloc(**kw) == status
    assert msg in last_error()


def test_chunk_noalloc_largest_accepted_sizes_pass_validation():
    """The scratch bound at Dk = Dv = 128 with bf16 inputs: 1807 sequence-heads with s_final, 960 without
    (the validation tests above reject one more; accepting calls need a device, so only the bound
    itself is checked here)."""
    assert (128 << 20) // 74240 == 1807
    assert ((128 << 20) - 960 * 65536) // 74240 >= 960 and ((128 << 20) - 961 * 65536) // 74240 < 961


def test_chunk_noalloc_nothing_to_do_returns_ok():
    assert chunk_noalloc(q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == 0
    assert chunk_noalloc(B=0) == 0


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, N=2, total=100, s0=None, o=FAKE, s_final=None, H=2,
             Dk=128, Dv=128, chunk=64, dtype=1, prologue=None, workspace=None, workspace_bytes=0, stream=None)
    a.update(kw)
    return kda.varlen_fwd_raw(*a.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(cu=None), 1, "cu_seqlens"), (dict(N=-1), 2, "N"), (dict(total=-5), 2, "total"),
    (dict(total=1 << 31), 2, "int32"), (dict(Dk=48), 2, "Dk"), (dict(chunk=128), 2, "chunk"),
    (dict(o=FAKE + 4), 4, "o"), (dict(dtype=-1), 3, "dtype"), (dict(g=None), 1, "g"),
    (dict(workspace=FAKE, workspace_bytes=(100 // 64 + 2) * 2 * 74240 - 1), 2, "workspace"),
])
def test_varlen_validation(kw, status, msg):
    assert varlen(**kw) == status
    assert msg in last_error()


def record_bytes(Dk, dtype):
    """Operand record of one (chunk, head).  fp32 inputs: Qt, Kt, Kbar^T as fp32 (4 B/value), six
    2 KiB fragments each of M^{-1} Diag(b) and of P, gamma_C (fp32).  bf16 inputs: -W, Qh, Kbar^T as
    fp16 (2 B/value), M^{-1} Diag(b) and P as six fp16 hi + lo fragment pairs (2 KiB each), gamma_C."""
    per_value = 12 if dtype == 0 else 6
    return 64 * Dk * per_value + 2 * 6 * 2048 + 4 * Dk


def test_record_sizes():
    assert record_bytes(128, 1) == 74240 and record_bytes(128, 0) == 123392
    assert record_bytes(64, 1) == 49408 and record_bytes(64, 0) == 73984


def segments(B, T, H, Dv):
    """Split-T segments: equal-length batches whose chain fills under half of 256 workgroups are cut
    so that the output pass has about 256 workgroups, segments of at least 64 chunks."""
    slices = B * H * (Dv // 32)
    if 2 * slices > 256:
        return 1
    P = min(256 // slices, (-(-T // 64)) // 64)
    return P if P >= 2 else 1


def segment_bytes(B, H, Dk, Dv, P):
    return 0 if P < 2 else B * H * Dk * 4 * ((P - 1) * (Dv + Dk) + P * Dv)


SPLIT_WINDOW_BUDGET = 3 << 30  # records of one T-window of a long split call (bf16 inputs)


def window_chunks(B, T, H, Dk, Dv, dtype, budget=SPLIT_WINDOW_BUDGET):
    """Chunks per T-window, or 0 for one piece: bf16 split calls whose records exceed the budget run
    as equal windows of at most the budget each."""
    nch = -(-T // 64)
    per_chunk = B * H * record_bytes(Dk, dtype)
    if dtype != 1 or segments(B, T, H, Dv) < 2 or nch * per_chunk <= budget:
        return 0
    wmax = max(budget // per_chunk, 1)
    nwin = -(-nch // wmax)
    return -(-nch // nwin)


def workspace_bytes(B, T, H, Dk, Dv, dtype, budget=SPLIT_WINDOW_BUDGET):
    W = window_chunks(B, T, H, Dk, Dv, dtype, budget)
    if W == 0:
        return B * (-(-T // 64)) * H * record_bytes(Dk, dtype) + segment_bytes(B, H, Dk, Dv, segments(B, T, H, Dv))
    state = -(-(B * H * Dk * Dv * 4) // 256) * 256  # carried between windows
    return state + B * W * H * record_bytes(Dk, dtype) + segment_bytes(B, H, Dk, Dv, segments(B, W * 64, H, Dv))


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("B,T,H,Dk,Dv", [(1, 64, 1, 128, 128), (4, 8192, 16, 128, 128), (2, 65, 3, 64, 128),
                                         (3, 1, 2, 64, 64), (1, 1 << 20, 8, 128, 128), (1, 16421, 2, 128, 128),
                                         (1, 8192, 1, 64, 64), (1, 1 << 19, 8, 128, 128)])
def test_chunk_workspace_size(B, T, H, Dk, Dv, dtype):
    assert kda.chunk_workspace_bytes(B, T, H, Dk, Dv, dtype) == workspace_bytes(B, T, H, Dk, Dv, dtype)


def test_long_split_calls_run_in_windows():
    # the million-token call: four windows of 4,096 chunks, 2.4 GB of records instead of 9.7 GB
    assert window_chunks(1, 1 << 20, 8, 128, 128, 1) == 4096
    assert kda.chunk_workspace_bytes(1, 1 << 20, 8, 128, 128) < 2.5e9
    assert window_chunks(4, 8192, 16, 128, 128, 1) == 0 and window_chunks(1, 1 << 20, 8, 128, 128, 0) == 0


def test_window_budget_override(monkeypatch):
    monkeypatch.setenv("KDA_SPLIT_WINDOW_BYTES", str(8 << 20))
    for B, T, H in [(1, 16421, 2), (1, 8192, 1), (1, 1 << 16, 2)]:
        assert kda.chunk_workspace_bytes(B, T, H, 128, 128) == workspace_bytes(B, T, H, 128, 128, 1, 8 << 20)
    assert window_chunks(1, 1 << 16, 2, 128, 128, 1, 8 << 20) > 0


def test_segment_counts():
    assert segments(1, 1 << 20, 8, 128) == 8 and segments(4, 8192, 16, 128) == 1
    assert segments(1, 16421, 2, 128) == 4 and segments(1, 8192, 1, 64) == 2


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("N,total,H,Dk", [(2, 100, 2, 128), (32, 65536, 16, 128), (1, 1, 1, 64)])
def test_varlen_workspace_size(N, total, H, Dk, dtype):
    order = -(-4 * N // 256) * 256  # the sequences' dispatch order, int32, 256-byte multiple
    assert kda.varlen_workspace_bytes(N, total, H, Dk, 128, dtype) == ((total // 64 + N) * H * record_bytes(Dk, dtype)
                                                                        + order)


def bwd_workspace_bytes(records, Dk, Dv):
    # the backward's workspace formula as the header states it: per record 4 (386 Dk + 20544 + 2 Dk Dv
    # + 192 Dv) bytes, plus one trash row of Dv floats in 256-byte granules
    return records * 4 * (386 * Dk + 20544 + 2 * Dk * Dv + 192 * Dv) + -(-(4 * Dv) // 256) * 256


@pytest.mark.parametrize("B,T,H,Dk,Dv", [(4, 8192, 16, 128, 128), (2, 200, 3, 64, 64), (1, 65, 2, 128, 64),
                                         (3, 100, 2, 64, 128), (1, 1, 1, 128, 64)])
def test_backward_workspace_size(B, T, H, Dk, Dv):
    assert kda.chunk_bwd_workspace_bytes(B, T, H, Dk, Dv) == bwd_workspace_bytes(B * -(-T // 64) * H, Dk, Dv)


@pytest.mark.parametrize("N,total,H,Dk", [(2, 100, 2, 128), (32, 65536, 16, 128), (3, 7, 1, 64)])
def test_varlen_backward_workspace_size(N, total, H, Dk):
    assert kda.varlen_bwd_workspace_bytes(N, total, H, Dk, 128) == bwd_workspace_bytes((total // 64 + N) * H, Dk, 128)


def test_workspace_size_of_unsupported_or_empty_is_zero():
    assert kda.chunk_workspace_bytes(0, 64, 1, 128, 128) == 0
    assert kda.chunk_workspace_bytes(1, 0, 1, 128, 128) == 0
    assert kda.chunk_workspace_bytes(1, 64, 1, 96, 128) == 0
    assert kda.chunk_workspace_bytes(1, 64, 1, 128, 128, 7) == 0
    assert kda.varlen_workspace_bytes(0, 10, 1, 128, 128) == 0


def test_varlen_nothing_to_do():
    assert varlen(N=0, cu=None) == 0


def decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s_in=FAKE, s_out=FAKE, o=FAKE, B=4, H=2, Dk=128, Dv=128,
             dtype=1, prologue=None, stream=None)
    a.update(kw)
    return kda.decode_step_raw(*a.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(s_in=None), 1, "s_in"), (dict(o=None), 1, "o"), (dict(Dv=100), 2, "Dv"), (dict(B=-1), 2, "B"),
    (dict(s_out=FAKE + 64), 2, "overlap"), (dict(k=FAKE + 2), 4, "k"), (dict(dtype=5), 3, "dtype"),
])
def test_decode_validation(kw, status, msg):
    assert decode(**kw) == status
    assert msg in last_error()


def test_decode_empty_batch_ok():
    assert decode(B=0, q=None, k=None, v=None, g=None, beta=None, s_in=None, s_out=None, o=None) == 0


def test_torch_front_end_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        kda.chunk_fwd(q, q, q, q.float(), torch.zeros(1, 64, 1))


def test_error_is_thread_local():
    import threading
    assert chunk(Dk=96) == 2
    seen = []
    t = threading.Thread(target=lambda: seen.append(last_error()))
    t.start()
    t.join()
    assert seen == [""] and "Dk" in last_error()


def test_prologue_validation():
    import ctypes
    bad = ctypes.pointer(kda.Prologue(5, 0, 0, 0, 0))
    assert chunk(prologue=bad) == 3 and "g_dtype" in last_error()
    bad = ctypes.pointer(kda.Prologue(0, 1, 9, 0, 0))
    assert varlen(prologue=bad) == 3 and "beta_dtype" in last_error()
    assert decode(prologue=bad) == 3 and "beta_dtype" in last_error()


def test_prologue_struct_defaults_to_none():
    import torch
    assert kda.prologue() is None
    p = kda.prologue(torch.bfloat16, True, torch.float32, False, True)
    assert (p.contents.g_dtype, p.contents.g_logit, p.contents.beta_dtype, p.contents.beta_logit,
            p.contents.qk_l2norm) == (1, 1, 0, 0, 1)


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library the binding raises; there is no fallback path to run instead."""
    monkeypatch.setattr(kda, "_LIB_PATH", os.path.join(ROOT, "no-such-dir", "libkda.so"))
    monkeypatch.setattr(kda, "_lib", None)
    with pytest.raises(ImportError, match="missing"):
        kda.load_library()
    with pytest.raises(ImportError):
        kda.chunk_workspace_bytes(1, 64, 1, 128, 128)
