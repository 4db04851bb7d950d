"""CPU oracle for the gated delta-rule (KDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the library under
``gated_delta_rule_65_amd`` never imports it, and this package imports
nothing from there.

``kda_oracle.c`` runs the recurrence token by token in fp64 (see its header
for the definition and the page it follows).  ``forward`` below only marshals
numpy arrays into it.

``prologue`` maps raw inputs to the recurrence's inputs in fp64: gate logits x
to log alpha = -softplus(x), beta logits b to 1 / (1 + e^-b), and q, k to unit
length per token and head.  The pages fix only the roles of alpha and beta and
the clamp of alpha to [e^-5, 1] (worldcybernews page "Kimi K3 Open Model
Surpasses Closed GPT and Anthropic Systems on Independent Benchmarks", second
paragraph); these logit forms are the customary parameterisation of such gates
and are written here from their definitions.

Parity status: pinned by ``tests/test_oracle_pins.py`` (hand-worked example,
exact rational arithmetic, dense brute force, closed forms, invariants) and,
for the prologue, by ``tests/test_oracle_prologue.py`` (closed-form values,
symmetries, and end-to-end reductions to runs with known gates).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle: gcc, IEEE fp64 (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
               _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def load(path: str):
    """Open an oracle shared library (the built one, or a test's variant of it)."""
    L = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.kda_oracle_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp, vp,
                                     ctypes.c_int]
    L.kda_oracle_forward.restype = ctypes.c_int
    L.kda_oracle_max_threads.restype = ctypes.c_int
    L.kda_oracle_backward.argtypes = [vp] * 8 + [vp, i64, i64, i64, i64] + [vp] * 6 + [ctypes.c_int]
    L.kda_oracle_backward.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load(_LIB)
    return _lib


def max_threads() -> int:
    return int(lib().kda_oracle_max_threads())


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def forward(q, k, v, g, beta, cu_seqlens, s0=None, cols: Optional[Sequence[int]] = None,
            want_state: bool = True, nthreads: int = 0, _lib=None):
    """Run the fp64 recurrence over packed sequences.

    q, k: [total, H, Dk]; v: [total, H, Dv]; g (log alpha, unclamped): [total, H, Dk];
    beta: [total, H]; cu_seqlens: [N+1]; s0: [N, H, Dk, Dv] or None.
    Inputs are taken as float64 (bf16 and fp32 values upcast exactly beforehand).
    cols: d_v columns to compute (default: all).
    Returns (o [total, H, ncols] float64, s_final [N, H, Dk, ncols] float64 or None).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    beta = _f64(beta)
    total, H, Dk = q.shape
    Dv = v.shape[2]
    if k.shape != (total, H, Dk) or g.shape != (total, H, Dk) or v.shape[:2] != (total, H) \
            or beta.shape != (total, H):
        raise ValueError("shape mismatch")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    if cu[0] != 0 or cu[-1] != total:
        raise ValueError("cu_seqlens must start at 0 and end at the token count")
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (N, H, Dk, Dv):
            raise ValueError("s0 shape")
    cols = np.arange(Dv, dtype=np.int32) if cols is None else np.ascontiguousarray(cols, dtype=np.int32)
    nc = cols.shape[0]
    o = np.zeros((total, H, nc), dtype=np.float64)
    sf = np.zeros((N, H, Dk, nc), dtype=np.float64) if want_state else None
    rc = (_lib or lib()).kda_oracle_forward(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(s0), _p(cu), N, H, Dk, Dv,
                                  _p(cols), nc, _p(o), _p(sf), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed ({rc})")
    return o, sf


def backward(q, k, v, g, beta, cu_seqlens, d_o, s0=None, d_sfinal=None, nthreads: int = 0, _lib=None):
    """Gradients of L with dL/do = d_o and dL/dS_T = d_sfinal (None = 0), in fp64.

    Shapes as for ``forward``; d_o: [total, H, Dv]; d_sfinal: [N, H, Dk, Dv] or None.
    Returns dict(dq, dk, dv, dg, dbeta, ds0) (dg is with respect to g = log alpha before the clamp)."""
    q, k, v, g, beta, d_o = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(d_o)
    total, H, Dk = q.shape
    Dv = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    if cu[0] != 0 or cu[-1] != total or d_o.shape != (total, H, Dv):
        raise ValueError("shape mismatch")
    s0 = None if s0 is None else _f64(s0)
    d_sfinal = None if d_sfinal is None else _f64(d_sfinal)
    out = dict(dq=np.zeros((total, H, Dk)), dk=np.zeros((total, H, Dk)), dv=np.zeros((total, H, Dv)),
               dg=np.zeros((total, H, Dk)), dbeta=np.zeros((total, H)), ds0=np.zeros((N, H, Dk, Dv)))
    rc = (_lib or lib()).kda_oracle_backward(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(s0), _p(d_o), _p(d_sfinal),
                                             _p(cu), N, H, Dk, Dv, _p(out["dq"]), _p(out["dk"]), _p(out["dv"]),
                                             _p(out["dg"]), _p(out["dbeta"]), _p(out["ds0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed ({rc})")
    return out


def softplus(x):
    """ln(1 + e^x), evaluated as max(x, 0) + ln(1 + e^-|x|) so that no exponential overflows."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x), evaluated through e^-|x| so that no exponential overflows."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def unit_rows(x):
    """x / ||x|| along the last axis; an all-zero vector stays zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def prologue(q, k, g, beta, g_logit=False, beta_logit=False, qk_l2norm=False):
    """The recurrence's inputs (fp64) from raw ones: log alpha = -softplus(g) for gate logits,
    beta = sigmoid(beta) for beta logits, q and k scaled to unit length per token and head."""
    q, k, g, beta = _f64(q), _f64(k), _f64(g), _f64(beta)
    if g_logit:
        g = -softplus(g)
    if beta_logit:
        beta = sigmoid(beta)
    if qk_l2norm:
        q, k = unit_rows(q), unit_rows(k)
    return q, k, g, beta


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    """Parity metric against the oracle: max|x - ref| / RMS(ref) over the whole array
    (max|x| when ref is all zero)."""
    rms = float(np.sqrt(np.mean(np.square(ref, dtype=np.float64))))
    if rms == 0.0:
        return float(np.abs(x).max()) if x.size else 0.0
    return float(np.abs(x.astype(np.float64) - ref).max() / rms)


def forward_inputs(inp, cols=None, want_state=True, nthreads=0):
    """Oracle on a ``kda_inputs.Inputs`` bundle (its prologue flags applied first)."""
    sp = inp.spec
    q, k, g, beta = prologue(inp.as_f32("q"), inp.as_f32("k"), inp.as_f32("g"), inp.as_f32("beta"),
                             g_logit=sp.g_logit, beta_logit=sp.beta_logit, qk_l2norm=sp.qk_l2norm)
    return forward(q, k, inp.as_f32("v"), g, beta, inp.cu_seqlens,
                   s0=None if inp.s0 is None else inp.s0.astype(np.float64), cols=cols,
                   want_state=want_state, nthreads=nthreads)
