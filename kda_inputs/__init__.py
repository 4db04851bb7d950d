"""Seeded synthetic inputs for the gated delta-rule (KDA) forward pass.

This package only draws random numbers and shapes them into the workloads'
tensors; it holds none of the attention method's arithmetic (no decay, no
clamp, no state update).  Both the HIP path and the CPU oracle are fed from
the same host arrays produced here.

Random numbers come from Philox4x32-10 (Salmon et al., SC'11) in
``philox_gen.c``; element ``e`` of a tensor drawn with (seed, stream) is word
``e % 4`` of the block with counter ``e // 4``.  Normals use Box-Muller.

Workload recipes follow the distributions stated for the method's inputs:
q, k ~ N(0,1) scaled to unit length per token; v ~ N(0,1); beta =
sigmoid(N(0,1)); log-alpha g = -softplus(N(0,1)) (the method clamps it, not
the generator); optional forcing of a fraction of g entries to the clamp
bounds; a long-memory regime g = -U(0, 0.01); initial states ~ N(0, std).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_gen.c")
_LIB = os.path.join(_HERE, "libkdagen.so")

# Stream ids: one independent Philox stream per tensor.
STREAM_Q, STREAM_K, STREAM_V, STREAM_BETA, STREAM_G, STREAM_GSEL, STREAM_S0, STREAM_LEN = range(1, 9)


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
               _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u32, u64, dp, fp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p
        L.kdagen_philox4x32_10.argtypes = [dp, dp, dp]
        L.kdagen_raw_u32.argtypes = [u32, u32, u64, u64, dp]
        L.kdagen_uniform.argtypes = [u32, u32, u64, u64, dp]
        L.kdagen_normal.argtypes = [u32, u32, u64, u64, dp]
        L.kdagen_normal_f32.argtypes = [u32, u32, u64, u64, ctypes.c_double, fp]
        L.kdagen_unit_rows_f32.argtypes = [u32, u32, u64, u32, fp]
        L.kdagen_unit_rows_f32.restype = ctypes.c_int
        L.kdagen_f32_to_bf16.argtypes = [fp, u64, dp]
        L.kdagen_bf16_to_f32.argtypes = [dp, u64, fp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- primitives

def philox_block(counter: Sequence[int], key: Sequence[int]) -> np.ndarray:
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    lib().kdagen_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def raw_u32(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().kdagen_raw_u32(seed, stream, first, n, _ptr(out))
    return out


def uniform(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().kdagen_uniform(seed, stream, first, n, _ptr(out))
    return out


def normal(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().kdagen_normal(seed, stream, first, n, _ptr(out))
    return out


def normal_f32(seed: int, stream: int, n: int, scale: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().kdagen_normal_f32(seed, stream, first, n, float(scale), _ptr(out))
    return out


def unit_rows_f32(seed: int, stream: int, rows: int, width: int) -> np.ndarray:
    out = np.empty((rows, width), dtype=np.float32)
    rc = lib().kdagen_unit_rows_f32(seed, stream, rows, width, _ptr(out))
    if rc != 0:
        raise ValueError("width out of range")
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().kdagen_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().kdagen_bf16_to_f32(_ptr(b), b.size, _ptr(out))
    return out


# ---------------------------------------------------------------- workloads

@dataclass
class Spec:
    """Shape and distribution recipe of one synthetic forward-pass input.

    lengths: tokens per sequence (all equal for the batched layout).
    gate: 'softplus' (g = -softplus(N(0,1))), 'softplus_bounds' (the same with
          a fraction ``bound_frac`` of entries forced to g=-5 or g=0, half
          each), 'longmem' (g = -U(0, 0.01)).
    s0_std: None for a zero initial state, else N(0, s0_std) entries.
    Raw-input forms (what the method's input prologue takes):
    g_logit: g holds the gate logits x ~ N(0, logit_std) themselves (gate 'softplus' only);
    beta_logit: beta holds its logits ~ N(0, 1); qk_l2norm: q and k are left at their
    N(0, 1) draws, not scaled to unit length; gate_dtype: 'f32' or 'bf16' storage of g and beta.
    """
    lengths: Sequence[int]
    H: int
    Dk: int
    Dv: int
    dtype: str = "bf16"            # 'bf16' or 'f32' (q, k, v and o)
    gate: str = "softplus"
    bound_frac: float = 0.05
    s0_std: Optional[float] = None
    seed: int = 0
    packed: bool = False           # packed varlen layout with cu_seqlens
    name: str = ""
    g_logit: bool = False
    beta_logit: bool = False
    qk_l2norm: bool = False
    logit_std: float = 1.0
    gate_dtype: str = "f32"

    @property
    def total(self) -> int:
        return int(sum(self.lengths))

    @property
    def n_seq(self) -> int:
        return len(self.lengths)


@dataclass
class Inputs:
    spec: Spec
    q: np.ndarray            # [sumL, H, Dk]  uint16 bf16 bits or float32
    k: np.ndarray            # [sumL, H, Dk]
    v: np.ndarray            # [sumL, H, Dv]
    g: np.ndarray            # [sumL, H, Dk]  float32 (or bf16 bits) log-alpha (unclamped), or gate logits
    beta: np.ndarray         # [sumL, H]      float32 (or bf16 bits), or logits
    s0: Optional[np.ndarray]  # [N, H, Dk, Dv] float32 or None
    cu_seqlens: np.ndarray   # [N+1] int32
    extra: dict = field(default_factory=dict)

    def as_f32(self, name: str) -> np.ndarray:
        """q/k/v/g/beta as float32 (exact upcast of the bf16 values)."""
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        return a


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def generate(spec: Spec) -> Inputs:
    L, H, Dk, Dv, s = spec.total, spec.H, spec.Dk, spec.Dv, spec.seed
    if spec.qk_l2norm:
        q = normal_f32(s, STREAM_Q, L * H * Dk).reshape(L, H, Dk)
        k = normal_f32(s, STREAM_K, L * H * Dk).reshape(L, H, Dk)
    else:
        q = unit_rows_f32(s, STREAM_Q, L * H, Dk).reshape(L, H, Dk)
        k = unit_rows_f32(s, STREAM_K, L * H, Dk).reshape(L, H, Dk)
    v = normal_f32(s, STREAM_V, L * H * Dv).reshape(L, H, Dv)
    if spec.dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif spec.dtype != "f32":
        raise ValueError(spec.dtype)
    if spec.beta_logit:
        beta = normal(s, STREAM_BETA, L * H).astype(np.float32).reshape(L, H)
    else:
        beta = _sigmoid(normal(s, STREAM_BETA, L * H)).astype(np.float32).reshape(L, H)
    n_g = L * H * Dk
    if spec.g_logit:
        if spec.gate != "softplus":
            raise ValueError("gate logits are drawn for the 'softplus' gate only")
        g = (spec.logit_std * normal(s, STREAM_G, n_g)).astype(np.float32)
    elif spec.gate in ("softplus", "softplus_bounds"):
        g = (-_softplus(normal(s, STREAM_G, n_g))).astype(np.float32)
        if spec.gate == "softplus_bounds":
            u = uniform(s, STREAM_GSEL, n_g)
            half = spec.bound_frac / 2.0
            g[u < half] = -5.0
            g[(u >= half) & (u < spec.bound_frac)] = 0.0
    elif spec.gate == "longmem":
        g = (-0.01 * uniform(s, STREAM_G, n_g)).astype(np.float32)
    else:
        raise ValueError(spec.gate)
    g = g.reshape(L, H, Dk)
    if spec.gate_dtype == "bf16":
        g, beta = f32_to_bf16_bits(g), f32_to_bf16_bits(beta)
    elif spec.gate_dtype != "f32":
        raise ValueError(spec.gate_dtype)
    s0 = None
    if spec.s0_std is not None:
        s0 = normal_f32(s, STREAM_S0, spec.n_seq * H * Dk * Dv, scale=spec.s0_std).reshape(spec.n_seq, H, Dk, Dv)
    cu = np.zeros(spec.n_seq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(spec.lengths, dtype=np.int64))
    return Inputs(spec, q, k, v, g, beta, s0, cu)


def loguniform_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    """floor(exp(U(ln lo, ln hi))) per sequence."""
    u = uniform(seed, STREAM_LEN, n)
    return [int(math.floor(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u]


# The five named workloads of the forward pass.
def workload(name: str) -> Spec:
    if name == "chunk_b1_h1_t256_d64_f32":
        return Spec([256], 1, 64, 64, "f32", "softplus", seed=0, name=name)
    if name == "chunk_b4_h16_t8192_d128_bf16":
        return Spec([8192] * 4, 16, 128, 128, "bf16", "softplus_bounds", 0.05, seed=1, name=name)
    if name == "varlen_n32_h16_d128_bf16":
        return Spec(loguniform_lengths(2, 32, 64, 16384), 16, 128, 128, "bf16", "softplus",
                    s0_std=0.02, seed=2, packed=True, name=name)
    if name == "decode_b256_h32_d128_bf16":
        return Spec([1] * 256, 32, 128, 128, "bf16", "softplus", s0_std=0.02, seed=3, name=name)
    if name == "prefill_b1_h8_t1m_d128_bf16":
        return Spec([1 << 20], 8, 128, 128, "bf16", "longmem", seed=4, name=name)
    raise KeyError(name)


WORKLOADS = ["chunk_b1_h1_t256_d64_f32", "chunk_b4_h16_t8192_d128_bf16", "varlen_n32_h16_d128_bf16",
             "decode_b256_h32_d128_bf16", "prefill_b1_h8_t1m_d128_bf16"]
