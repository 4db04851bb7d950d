"""Shared helpers for the GPU tests: move generator output to the device, compare
against the oracle with the max|err| / RMS metric."""
import numpy as np
import torch

import kda_inputs

TOL = {"bf16": 2e-2, "f32": 1e-4}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, shape=None) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    if shape is not None:
        t = t.reshape(shape)
    return t.to(dev())


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.square(ref, dtype=np.float64))))
    if rms == 0.0:
        return float(np.abs(gpu).max()) if gpu.size else 0.0
    return float(np.abs(gpu.astype(np.float64) - ref).max() / rms)


def device_inputs(inp: kda_inputs.Inputs, batched: bool):
    """Device tensors for the chunk entry point (batched [B,T,H,D]) or varlen ([total,H,D])."""
    sp = inp.spec
    if batched:
        B, T = sp.n_seq, sp.lengths[0]
        assert all(L == T for L in sp.lengths)
        sh_k, sh_v, sh_b = (B, T, sp.H, sp.Dk), (B, T, sp.H, sp.Dv), (B, T, sp.H)
    else:
        sh_k, sh_v, sh_b = inp.q.shape, inp.v.shape, inp.beta.shape
    d = dict(q=to_dev(inp.q, sh_k), k=to_dev(inp.k, sh_k), v=to_dev(inp.v, sh_v), g=to_dev(inp.g, sh_k),
             beta=to_dev(inp.beta, sh_b))
    d["s0"] = None if inp.s0 is None else to_dev(inp.s0)
    if not batched:
        d["cu_seqlens"] = to_dev(inp.cu_seqlens.astype(np.int32))
    return d
