"""Gated delta-rule (Kimi Delta Attention) forward pass on AMD MI355X (gfx950).

A thin ctypes binding over ``libkda.so`` (C ABI in ``include/kda.h``).  Every
step of the computation runs in the library's HIP kernels; this module only
checks tensor properties, allocates outputs with torch and passes raw device
pointers plus torch's current HIP stream.  There is no fallback: if the library
is missing or the tensors are not on a GPU, the call raises.

Recurrence per head (worldcybernews page "Kimi K3 Open Model Surpasses Closed
GPT and Anthropic Systems on Independent Benchmarks", second paragraph, read as
the gated delta rule):  S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
o_t = S_t^T q_t, a_t = exp(clamp(g_t, -5, 0)).

Input prologue (every entry point): g and beta may be float32 or bfloat16;
``g_logit=True`` reads g as gate logits x with log a = -softplus(x);
``beta_logit=True`` reads beta as logits (b = sigmoid(beta)); ``qk_l2norm=True``
scales q and k to unit length per token and head inside the kernels.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_noalloc_raw", "varlen_fwd", "decode_step", "library_path", "load_library", "KDAError",
           "chunk_fwd_raw", "varlen_fwd_raw", "decode_step_raw", "chunk_workspace_bytes",
           "varlen_workspace_bytes", "DTYPE", "Prologue", "prologue", "chunk_bwd", "varlen_bwd", "chunk_bwd_raw",
           "varlen_bwd_raw", "chunk_bwd_workspace_bytes", "varlen_bwd_workspace_bytes", "ChunkKDA",
           "calib_copy_raw", "calib_mfma_raw"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
DTYPE = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}
STATUS = {0: "OK", 1: "NULL_ARG", 2: "BAD_SHAPE", 3: "BAD_DTYPE", 4: "MISALIGNED", 5: "HIP_ERROR"}


class Prologue(ctypes.Structure):
    """kda_prologue of the C ABI."""
    _fields_ = [("g_dtype", ctypes.c_int), ("g_logit", ctypes.c_int), ("beta_dtype", ctypes.c_int),
                ("beta_logit", ctypes.c_int), ("qk_l2norm", ctypes.c_int)]


def prologue(g_dtype=torch.float32, g_logit=False, beta_dtype=torch.float32, beta_logit=False, qk_l2norm=False):
    """A ctypes pointer to a kda_prologue, or None when every field has its default."""
    codes = (_dtype_code(g_dtype), int(bool(g_logit)), _dtype_code(beta_dtype), int(bool(beta_logit)),
             int(bool(qk_l2norm)))
    if codes == (KDA_F32, 0, KDA_F32, 0, 0):
        return None
    return ctypes.pointer(Prologue(*codes))


class KDAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kda status {status} ({STATUS.get(status, '?')}): {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


_lib = None


def load_library():
    """Open libkda.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                          f"g.build()'` or `python gated_delta_rule_65_amd/_build.py`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    pp = ctypes.POINTER(Prologue)
    L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, ci, ci, ci, ci, pp, vp, sz, vp]
    L.kda_chunk_fwd.restype = ci
    L.kda_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, ci, ci, ci, ci, ci, pp, vp, sz, vp]
    L.kda_varlen_fwd.restype = ci
    L.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, ci, ci, ci, ci, pp, vp]
    L.kda_chunk_fwd_noalloc.restype = ci
    L.kda_chunk_workspace_bytes.argtypes = [i64, i64, ci, ci, ci, ci]
    L.kda_chunk_workspace_bytes.restype = sz
    L.kda_varlen_workspace_bytes.argtypes = [i64, i64, ci, ci, ci, ci]
    L.kda_varlen_workspace_bytes.restype = sz
    L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, ci, ci, ci, ci, pp, vp]
    L.kda_decode_step.restype = ci
    L.kda_chunk_bwd.argtypes = [vp] * 14 + [i64, i64, ci, ci, ci, ci, ci, vp, sz, vp]
    L.kda_chunk_bwd.restype = ci
    L.kda_varlen_bwd.argtypes = [vp] * 6 + [i64, i64] + [vp] * 9 + [ci, ci, ci, ci, ci, vp, sz, vp]
    L.kda_varlen_bwd.restype = ci
    L.kda_chunk_bwd_workspace_bytes.argtypes = [i64, i64, ci, ci, ci, ci]
    L.kda_chunk_bwd_workspace_bytes.restype = sz
    L.kda_varlen_bwd_workspace_bytes.argtypes = [i64, i64, ci, ci, ci, ci]
    L.kda_varlen_bwd_workspace_bytes.restype = sz
    L.kda_calib_copy.argtypes = [vp, vp, sz, vp]
    L.kda_calib_copy.restype = ci
    L.kda_calib_mfma.argtypes = [vp, ci, i64, ci, vp]
    L.kda_calib_mfma.restype = ci
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise KDAError(status, load_library().kda_last_error().decode())


# ----------------------------------------------------------------- raw calls (ints in, status out)

def chunk_fwd_raw(q, k, v, g, beta, s0, o, s_final, B, T, H, Dk, Dv, chunk, dtype, prologue, workspace,
                  workspace_bytes, stream) -> int:
    return load_library().kda_chunk_fwd(q, k, v, g, beta, s0, o, s_final, B, T, H, Dk, Dv, chunk, dtype, prologue,
                                        workspace, workspace_bytes, stream)


def chunk_fwd_noalloc_raw(q, k, v, g, beta, s0, o, s_final, B, T, H, Dk, Dv, chunk, dtype, prologue, stream) -> int:
    return load_library().kda_chunk_fwd_noalloc(q, k, v, g, beta, s0, o, s_final, B, T, H, Dk, Dv, chunk, dtype,
                                                prologue, stream)


def varlen_fwd_raw(q, k, v, g, beta, cu, N, total, s0, o, s_final, H, Dk, Dv, chunk, dtype, prologue, workspace,
                   workspace_bytes, stream) -> int:
    return load_library().kda_varlen_fwd(q, k, v, g, beta, cu, N, total, s0, o, s_final, H, Dk, Dv, chunk, dtype,
                                         prologue, workspace, workspace_bytes, stream)


def calib_copy_raw(src, dst, nbytes, stream) -> int:
    """kda_calib_copy: a plain device copy of nbytes (the achievable HBM rate)."""
    return load_library().kda_calib_copy(src, dst, nbytes, stream)


def calib_mfma_raw(out, blocks, iters, kind, stream) -> int:
    """kda_calib_mfma: a dense bf16 matrix-core loop (kind 0: 16x16x32, kind 1: 32x32x16)."""
    return load_library().kda_calib_mfma(out, blocks, iters, kind, stream)


def _dtype_code(dtype) -> int:
    return DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)


def chunk_workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, dtype=torch.bfloat16) -> int:
    return int(load_library().kda_chunk_workspace_bytes(B, T, H, Dk, Dv, _dtype_code(dtype)))


def varlen_workspace_bytes(N: int, total: int, H: int, Dk: int, Dv: int, dtype=torch.bfloat16) -> int:
    return int(load_library().kda_varlen_workspace_bytes(N, total, H, Dk, Dv, _dtype_code(dtype)))


def decode_step_raw(q, k, v, g, beta, s_in, s_out, o, B, H, Dk, Dv, dtype, prologue, stream) -> int:
    return load_library().kda_decode_step(q, k, v, g, beta, s_in, s_out, o, B, H, Dk, Dv, dtype, prologue, stream)


def chunk_bwd_raw(q, k, v, g, beta, s0, d_o, d_sfinal, dq, dk, dv, dg, dbeta, ds0, B, T, H, Dk, Dv, chunk, dtype,
                  workspace, workspace_bytes, stream) -> int:
    return load_library().kda_chunk_bwd(q, k, v, g, beta, s0, d_o, d_sfinal, dq, dk, dv, dg, dbeta, ds0, B, T, H, Dk,
                                        Dv, chunk, dtype, workspace, workspace_bytes, stream)


def varlen_bwd_raw(q, k, v, g, beta, cu, N, total, s0, d_o, d_sfinal, dq, dk, dv, dg, dbeta, ds0, H, Dk, Dv, chunk,
                   dtype, workspace, workspace_bytes, stream) -> int:
    return load_library().kda_varlen_bwd(q, k, v, g, beta, cu, N, total, s0, d_o, d_sfinal, dq, dk, dv, dg, dbeta,
                                         ds0, H, Dk, Dv, chunk, dtype, workspace, workspace_bytes, stream)


def chunk_bwd_workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, dtype=torch.bfloat16) -> int:
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, _dtype_code(dtype)))


def varlen_bwd_workspace_bytes(N: int, total: int, H: int, Dk: int, Dv: int, dtype=torch.bfloat16) -> int:
    return int(load_library().kda_varlen_bwd_workspace_bytes(N, total, H, Dk, Dv, _dtype_code(dtype)))


# ----------------------------------------------------------------- torch front end

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _gates(g, beta, g_shape, b_shape, g_logit, beta_logit, qk_l2norm):
    """Check g and beta (float32 or bfloat16 each) and build the prologue for them."""
    for t, name, shape in ((g, "g", g_shape), (beta, "beta", b_shape)):
        if t.dtype not in DTYPE:
            raise TypeError(f"{name} must be float32 or bfloat16 (got {t.dtype})")
        _need(t, name, t.dtype, shape)
    return prologue(g.dtype, g_logit, beta.dtype, beta_logit, qk_l2norm)


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _workspace(need: int, fused: bool, workspace: Optional[torch.Tensor], device
               ) -> Tuple[Optional[torch.Tensor], int]:
    """Pointer and size of the workspace to pass: none for the fused kernel, the caller's buffer,
    or a fresh torch allocation (torch's caching allocator makes that cheap)."""
    if fused or need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    else:
        _need(workspace, "workspace")
        if workspace.device != device:
            raise ValueError("workspace must be on the same GPU as q")
    return workspace, workspace.numel() * workspace.element_size()


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              s0: Optional[torch.Tensor] = None, chunk: int = 64, output_final_state: bool = True,
              fused: bool = False, workspace: Optional[torch.Tensor] = None, g_logit: bool = False,
              beta_logit: bool = False, qk_l2norm: bool = False
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill over equal-length sequences.

    q, k: [B, T, H, Dk]; v: [B, T, H, Dv] (bf16 or fp32, all the same);
    g (log forget gate, or gate logits with ``g_logit``; fp32 or bf16): [B, T, H, Dk];
    beta (fp32 or bf16; logits with ``beta_logit``): [B, T, H]; s0 (fp32): [B, H, Dk, Dv] or None.
    ``qk_l2norm`` scales q and k to unit length per token and head inside the kernels.
    Returns o (fp32) [B, T, H, Dv] and the final state [B, H, Dk, Dv] (or None).
    By default the two-kernel path runs with a workspace (``workspace`` if given, else allocated);
    ``fused=True`` selects the single fused kernel, which needs none.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, Dk]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in DTYPE:
        raise TypeError("q/k/v must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    pro = _gates(g, beta, (B, T, H, Dk), (B, T, H), g_logit, beta_logit, qk_l2norm)
    if s0 is not None:
        _need(s0, "s0", torch.float32, (B, H, Dk, Dv))
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    sf = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if output_final_state else None
    ws, ws_bytes = _workspace(chunk_workspace_bytes(B, T, H, Dk, Dv, q.dtype), fused, workspace, q.device)
    with torch.cuda.device(q.device):
        _check(chunk_fwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o), _ptr(sf),
                             B, T, H, Dk, Dv, chunk, DTYPE[q.dtype], pro, _ptr(ws), ws_bytes, _stream(q.device)))
    return o, sf


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                      s0: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                      s_final: Optional[torch.Tensor] = None, g_logit: bool = False, beta_logit: bool = False,
                      qk_l2norm: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """:func:`chunk_fwd` through the library's fixed per-GPU scratch (no workspace, nothing
    allocated by the library).  Pass preallocated ``o`` [B, T, H, Dv] (fp32) and ``s_final``
    [B, H, Dk, Dv] (fp32, or None for no final state) to allocate nothing here either; if ``o`` is
    None it is allocated with torch.  Calls on one GPU share the scratch and must not overlap."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, Dk]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in DTYPE:
        raise TypeError("q/k/v must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    pro = _gates(g, beta, (B, T, H, Dk), (B, T, H), g_logit, beta_logit, qk_l2norm)
    if s0 is not None:
        _need(s0, "s0", torch.float32, (B, H, Dk, Dv))
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32, (B, T, H, Dv))
    if s_final is not None:
        _need(s_final, "s_final", torch.float32, (B, H, Dk, Dv))
    with torch.cuda.device(q.device):
        _check(chunk_fwd_noalloc_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o),
                                     _ptr(s_final), B, T, H, Dk, Dv, 64, DTYPE[q.dtype], pro, _stream(q.device)))
    return o, s_final


def varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
               cu_seqlens: torch.Tensor, s0: Optional[torch.Tensor] = None, chunk: int = 64,
               output_final_state: bool = True, fused: bool = False, workspace: Optional[torch.Tensor] = None,
               g_logit: bool = False, beta_logit: bool = False, qk_l2norm: bool = False
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Packed variable-length prefill.

    q, k, g: [total, H, Dk]; v: [total, H, Dv]; beta: [total, H]; cu_seqlens: int32 [N+1] on the GPU;
    s0: [N, H, Dk, Dv] or None.  Returns o [total, H, Dv] (fp32) and the final states [N, H, Dk, Dv].
    ``fused``, ``workspace`` and the prologue options as for :func:`chunk_fwd`.
    """
    if q.dim() != 3:
        raise ValueError("q must be [total, H, Dk]")
    total, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in DTYPE:
        raise TypeError("q/k/v must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (total, H, Dk))
    _need(v, "v", q.dtype, (total, H, Dv))
    pro = _gates(g, beta, (total, H, Dk), (total, H), g_logit, beta_logit, qk_l2norm)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if s0 is not None:
        _need(s0, "s0", torch.float32, (N, H, Dk, Dv))
    o = torch.empty((total, H, Dv), dtype=torch.float32, device=q.device)
    sf = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device) if output_final_state else None
    ws, ws_bytes = _workspace(varlen_workspace_bytes(N, total, H, Dk, Dv, q.dtype), fused, workspace, q.device)
    with torch.cuda.device(q.device):
        _check(varlen_fwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, total,
                              _ptr(s0), _ptr(o), _ptr(sf), H, Dk, Dv, chunk, DTYPE[q.dtype], pro, _ptr(ws),
                              ws_bytes, _stream(q.device)))
    return o, sf


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                state: torch.Tensor, inplace: bool = False, g_logit: bool = False, beta_logit: bool = False,
                qk_l2norm: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """One token per sequence.  q, k, g: [B, H, Dk]; v: [B, H, Dv]; beta: [B, H];
    state (fp32): [B, H, Dk, Dv].  Returns o [B, H, Dv] (fp32) and the new state
    (``state`` itself when ``inplace``).  Prologue options as for :func:`chunk_fwd`."""
    if q.dim() != 3:
        raise ValueError("q must be [B, H, Dk]")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in DTYPE:
        raise TypeError("q/k/v must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, H, Dk))
    _need(v, "v", q.dtype, (B, H, Dv))
    pro = _gates(g, beta, (B, H, Dk), (B, H), g_logit, beta_logit, qk_l2norm)
    _need(state, "state", torch.float32, (B, H, Dk, Dv))
    o = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    out_state = state if inplace else torch.empty_like(state)
    with torch.cuda.device(q.device):
        _check(decode_step_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out_state),
                               _ptr(o), B, H, Dk, Dv, DTYPE[q.dtype], pro, _stream(q.device)))
    return o, out_state


def _bwd_workspace(need: int, workspace: Optional[torch.Tensor], device) -> Tuple[Optional[torch.Tensor], int]:
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    else:
        _need(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              d_o: torch.Tensor, s0: Optional[torch.Tensor] = None, d_sfinal: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None):
    """Gradients of :func:`chunk_fwd` (g = log alpha and beta as given, fp32) for dL/do = d_o and
    dL/dS_T = d_sfinal (None = 0).  Returns dq, dk, dv, dg, dbeta, ds0 (all fp32); dg is with respect
    to g before the clamp."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, Dk]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in DTYPE:
        raise TypeError("q/k/v must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    _need(g, "g", torch.float32, (B, T, H, Dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(d_o, "d_o", torch.float32, (B, T, H, Dv))
    if s0 is not None:
        _need(s0, "s0", torch.float32, (B, H, Dk, Dv))
    if d_sfinal is not None:
        _need(d_sfinal, "d_sfinal", torch.float32, (B, H, Dk, Dv))
    f = dict(dtype=torch.float32, device=q.device)
    dq, dk, dg = (torch.empty((B, T, H, Dk), **f) for _ in range(3))
    dv = torch.empty((B, T, H, Dv), **f)
    dbeta = torch.empty((B, T, H), **f)
    ds0 = torch.empty((B, H, Dk, Dv), **f)
    ws, ws_bytes = _bwd_workspace(chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, q.dtype), workspace, q.device)
    with torch.cuda.device(q.device):
        _check(chunk_bwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(d_o), _ptr(d_sfinal),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(ds0), B, T, H, Dk, Dv, 64,
                             DTYPE[q.dtype], _ptr(ws), ws_bytes, _stream(q.device)))
    return dq, dk, dv, dg, dbeta, ds0


def varlen_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
               cu_seqlens: torch.Tensor, d_o: torch.Tensor, s0: Optional[torch.Tensor] = None,
               d_sfinal: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gradients of :func:`varlen_fwd`; layouts as there, results as for :func:`chunk_bwd`."""
    if q.dim() != 3:
        raise ValueError("q must be [total, H, Dk]")
    total, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in DTYPE:
        raise TypeError("q/k/v must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (total, H, Dk))
    _need(v, "v", q.dtype, (total, H, Dv))
    _need(g, "g", torch.float32, (total, H, Dk))
    _need(beta, "beta", torch.float32, (total, H))
    _need(d_o, "d_o", torch.float32, (total, H, Dv))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if s0 is not None:
        _need(s0, "s0", torch.float32, (N, H, Dk, Dv))
    if d_sfinal is not None:
        _need(d_sfinal, "d_sfinal", torch.float32, (N, H, Dk, Dv))
    f = dict(dtype=torch.float32, device=q.device)
    dq, dk, dg = (torch.empty((total, H, Dk), **f) for _ in range(3))
    dv = torch.empty((total, H, Dv), **f)
    dbeta = torch.empty((total, H), **f)
    ds0 = torch.empty((N, H, Dk, Dv), **f)
    ws, ws_bytes = _bwd_workspace(varlen_bwd_workspace_bytes(N, total, H, Dk, Dv, q.dtype), workspace, q.device)
    with torch.cuda.device(q.device):
        _check(varlen_bwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, total, _ptr(s0),
                              _ptr(d_o), _ptr(d_sfinal), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                              _ptr(ds0), H, Dk, Dv, 64, DTYPE[q.dtype], _ptr(ws), ws_bytes, _stream(q.device)))
    return dq, dk, dv, dg, dbeta, ds0


class ChunkKDA(torch.autograd.Function):
    """Autograd wrapper: ``o, s_final = ChunkKDA.apply(q, k, v, g, beta, s0)`` with the forward and
    backward both in the library's kernels.  Gradients of q, k, v come back in fp32 and are cast
    to the input type; s0 may be None."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, s0=None):
        o, sf = chunk_fwd(q, k, v, g, beta, s0)
        ctx.save_for_backward(q, k, v, g, beta, s0)
        return o, sf

    @staticmethod
    def backward(ctx, d_o, d_sf):
        q, k, v, g, beta, s0 = ctx.saved_tensors
        d_o = torch.zeros_like(q[..., :1].float()).expand(*q.shape[:-1], v.shape[-1]).contiguous() \
            if d_o is None else d_o.float().contiguous()
        d_sf = None if d_sf is None else d_sf.float().contiguous()
        dq, dk, dv, dg, dbeta, ds0 = chunk_bwd(q, k, v, g, beta, d_o, s0, d_sf)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dg, dbeta, (ds0 if s0 is not None else None)
