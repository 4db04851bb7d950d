"""CPU oracle for the gated delta-rule (KDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the library under
``gated_delta_rule_65_amd`` never imports it, and this package imports
nothing from there.

``kda_oracle.c`` runs the recurrence token by token in fp64 (see its header
for the definition and the page it follows).  ``forward`` below only marshals
numpy arrays into it.

Parity status: pinned by ``tests/test_oracle_pins.py`` (hand-worked example,
exact rational arithmetic, dense brute force, closed forms, invariants).
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


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def forward(q, k, v, g, beta, cu_seqlens, s0=None, cols: Optional[Sequence[int]] = None,
            want_state: bool = True, nthreads: int = 0, _lib=None):
    """Run the fp64 recurrence over packed sequences.

    q, k: [total, H, Dk]; v: [total, H, Dv]; g (log alpha, unclamped): [total, H, Dk];
    beta: [total, H]; cu_seqlens: [N+1]; s0: [N, H, Dk, Dv] or None.
    Inputs are taken as float32 (bf16 values upcast exactly beforehand).
    cols: d_v columns to compute (default: all).
    Returns (o [total, H, ncols] float64, s_final [N, H, Dk, ncols] float64 or None).
    """
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    beta = _f32(beta)
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


def forward_inputs(inp, cols=None, want_state=True, nthreads=0):
    """Oracle on a ``kda_inputs.Inputs`` bundle."""
    return forward(inp.as_f32("q"), inp.as_f32("k"), inp.as_f32("v"), inp.g, inp.beta, inp.cu_seqlens,
                   s0=None if inp.s0 is None else inp.s0.astype(np.float64), cols=cols,
                   want_state=want_state, nthreads=nthreads)
