"""Throughput benchmark of the gated delta-rule (KDA) forward pass on one MI355X.

Timed step: one kda_chunk_fwd call over the chunked-prefill batch B=4, H=16,
T=8192, d_k=d_v=128 (bf16 q/k/v, fp32 gates, fp32 state and output), inputs
and the workspace resident in HBM (the call launches the per-chunk preparation
kernel and the state-chain kernel).  value = B*T tokens per step / seconds per step.

Also reported on the same JSON line:
  roofline      the call's two kernels against HBM bandwidth (algorithmic bytes / time)
  mfma          the same call's algorithmic FLOPs against the dense bf16 MFMA peak
  fused         the single fused kernel (workspace NULL) on the same batch
  decode        single-token decode step, B=256, H=32, d=128: GB/s against HBM peak
  varlen        packed varlen prefill, 32 sequences, H=16, d=128: tokens/s
  cpu_baseline  the fp64 CPU oracle on the same chunked batch (rank 0 only)
  parity        max|err|/RMS of the timed output against that oracle run

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def chunk_alg_bytes(n_head_tokens, n_heads, Dk, Dv, in_bytes, with_s0, gate_bytes=4):
    # q, k, v in the input type; g (Dk) and beta in the gate type (fp32 unless given); o fp32 (Dv);
    # final state fp32 (+ initial state if given)
    per_tok = (2 * Dk + Dv) * in_bytes + gate_bytes * (Dk + 1) + 4 * Dv
    return n_head_tokens * per_tok + n_heads * Dk * Dv * 4 * (2 if with_s0 else 1)


def chunk_alg_flops(n_head_tokens, Dk, Dv, C=64):
    # three state products, two triangular Gram matrices, triangular P.U, triangular solve on [K|V]
    return n_head_tokens * (6 * Dk * Dv + 2 * C * Dk + C * Dv + C * (Dk + Dv))


def decode_alg_bytes(B, H, Dk, Dv, in_bytes):
    return B * H * (2 * Dk * Dv * 4 + (2 * Dk + Dv) * in_bytes + 4 * Dk + 4 + 4 * Dv)


def kernel_source_digest():
    """Digest of the kernel sources with comments and blank space removed, so that the recorded
    counters stay attached to the code they were measured on and only a code change drops them."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_65_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)               # line comments (no string holds //)
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
    profiles/traffic.json, scaled by the same counters on a plain copy of known size.
    None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


def time_launches(fn, steps, warmup, torch):
    """Run fn warmup times, then `steps` times bracketed by synchronize; per-launch
    durations from events on the current stream (the stream the library launches on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in evs]
    return wall, float(np.mean(per)), float(np.min(per))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the GPU clock settles only after ~40 back-to-back calls (~25 ms of load); earlier calls run
    # up to 14% slower, so the default warm-up covers that ramp
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode and varlen measurements")
    ap.add_argument("--only", choices=["chunk", "decode", "varlen", "prefill_1m", "raw_gates", "backward"],
                    default=None,
                    help="time one workload only (for profiler runs); prints its own JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path runs on a single device.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_65_amd as kda
    import kda_inputs
    from tests.gpu_util import device_inputs, rel_err, to_dev

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kda.load_library()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 3}))
        return

    if args.only == "decode":
        print(json.dumps({"decode": measure_decode(args, torch, kda, kda_inputs, to_dev)}))
        return
    if args.only == "varlen":
        print(json.dumps({"varlen": measure_varlen(args, torch, kda, kda_inputs, device_inputs)}))
        return
    if args.only == "prefill_1m":
        print(json.dumps({"prefill_1m": measure_prefill_1m(args, torch, kda, kda_inputs, device_inputs)}))
        return
    if args.only == "backward":
        print(json.dumps({"backward": measure_backward(args, torch, kda, kda_inputs, device_inputs)}))
        return
    if args.only == "raw_gates":
        print(json.dumps({"raw_gates": measure_raw_gates(args, torch, kda, kda_inputs, device_inputs)}))
        return

    # ------------------------------------------------ chunked prefill, B=4 H=16 T=8192 d=128 bf16
    name = "chunk_b4_h16_t8192_d128_bf16"
    spec = kda_inputs.workload(name)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, batched=True)
    B, T, H, Dk, Dv = spec.n_seq, spec.lengths[0], spec.H, spec.Dk, spec.Dv
    out = {}
    ws = torch.empty(kda.chunk_workspace_bytes(B, T, H, Dk, Dv), dtype=torch.uint8, device="cuda")

    def step():
        out["o"], out["s"] = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], workspace=ws)

    def step_fused():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], fused=True)

    wall, k_ms, k_min = time_launches(step, args.steps, args.warmup, torch)
    ms_per_step = wall * 1e3 / args.steps
    tokens = B * T
    value = tokens * args.steps / wall
    n_ht = tokens * H
    alg_bytes = chunk_alg_bytes(n_ht, B * H, Dk, Dv, 2, with_s0=False)
    alg_flops = chunk_alg_flops(n_ht, Dk, Dv)
    gbs = alg_bytes / (k_ms * 1e-3) / 1e9
    tflops = alg_flops / (k_ms * 1e-3) / 1e12
    traffic = measured_traffic(name)

    line = {
        "metric": "KDA fwd tokens/s (H=16,d=128,T=8192) + % MFMA peak; decode % HBM BW",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "T": T, "H": H, "d_k": Dk, "d_v": Dv, "chunk": 64,
                   "qkv": "bf16", "gates": "fp32", "state": "fp32", "output": "fp32", "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "prep_kernel<128,false,false,false,false> + chain_kernel<128,false,false,false,false>", "kernel_ms": k_ms,
                     "kernel_ms_min": k_min, "alg_bytes_per_launch": alg_bytes,
                     "workspace_bytes": ws.numel()},
        "mfma": {"achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "alg_flops_per_launch": alg_flops},
    }
    if args.only is None and not args.no_extras:
        _, f_ms, f_min = time_launches(step_fused, max(10, args.steps // 2), args.warmup, torch)
        line["fused"] = {"kernel": "chunk_fwd_kernel<128,false>", "kernel_ms": f_ms, "kernel_ms_min": f_min,
                         "tokens_per_s": tokens / (f_ms * 1e-3),
                         "achieved": alg_bytes / (f_ms * 1e-3) / 1e9, "unit": "GB/s"}

    if args.only is None and not args.no_extras:
        line["decode"] = measure_decode(args, torch, kda, kda_inputs, to_dev)
        line["varlen"] = measure_varlen(args, torch, kda, kda_inputs, device_inputs)
        line["prefill_1m"] = measure_prefill_1m(args, torch, kda, kda_inputs, device_inputs)
        line["raw_gates"] = measure_raw_gates(args, torch, kda, kda_inputs, device_inputs)
        line["backward"] = measure_backward(args, torch, kda, kda_inputs, device_inputs)

    if args.only is None and not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        o_ref, s_ref = oracle.forward_inputs(inp)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                                "kind": "oracle", "seconds": dt,
                                "sample": f"the whole timed batch ({B}x{T} tokens, {H} heads, all {Dv} columns), "
                                          "fp64 token-by-token recurrence"}
        o_gpu = out["o"].reshape(tokens, H, Dv).cpu().numpy()
        line["parity"] = {"o_err": rel_err(o_gpu, o_ref), "s_err": rel_err(out["s"].cpu().numpy(), s_ref),
                          "tol": 2e-2, "metric": "max|err|/RMS vs fp64 oracle"}

    print(json.dumps(line))


def measure_decode(args, torch, kda, kda_inputs, to_dev):
    """Single-token decode step, B=256 H=32 d=128: GB/s of algorithmic bytes per launch."""
    name = "decode_b256_h32_d128_bf16"
    dspec = kda_inputs.workload(name)
    dinp = kda_inputs.generate(dspec)
    Bd, Hd = dspec.n_seq, dspec.H
    dq = to_dev(dinp.q, (Bd, Hd, 128))
    dk = to_dev(dinp.k, (Bd, Hd, 128))
    dv = to_dev(dinp.v, (Bd, Hd, 128))
    dg = to_dev(dinp.g, (Bd, Hd, 128))
    db = to_dev(dinp.beta, (Bd, Hd))
    s0 = to_dev(dinp.s0)
    st = [s0, torch.empty_like(s0)]
    flip = [0]
    o = torch.empty((Bd, Hd, 128), dtype=torch.float32, device=dq.device)

    def dstep():
        # ping-pong between two state buffers: every launch reads and writes a full state
        a = flip[0]
        rc = kda.decode_step_raw(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dg.data_ptr(), db.data_ptr(),
                                 st[a].data_ptr(), st[1 - a].data_ptr(), o.data_ptr(), Bd, Hd, 128, 128,
                                 kda.DTYPE[torch.bfloat16], None, torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        flip[0] = 1 - a

    _, dk_ms, dk_min = time_launches(dstep, max(20, args.steps), args.warmup, torch)
    dbytes = decode_alg_bytes(Bd, Hd, 128, 128, 2)
    dgbs = dbytes / (dk_ms * 1e-3) / 1e9
    return {"workload": name, "kernel_ms": dk_ms, "kernel_ms_min": dk_min, "achieved": dgbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS, "alg_bytes_per_launch": dbytes,
            "tokens_per_s": Bd / (dk_ms * 1e-3), "traffic": measured_traffic(name)}


def measure_varlen(args, torch, kda, kda_inputs, device_inputs):
    """Packed varlen prefill, 32 sequences (log-uniform lengths), H=16 d=128."""
    name = "varlen_n32_h16_d128_bf16"
    vspec = kda_inputs.workload(name)
    vinp = kda_inputs.generate(vspec)
    vd = device_inputs(vinp, batched=False)

    H, Dk, Dv = vspec.H, vspec.Dk, vspec.Dv
    ws = torch.empty(kda.varlen_workspace_bytes(vspec.n_seq, vspec.total, H, Dk, Dv), dtype=torch.uint8,
                     device="cuda")

    def vstep():
        kda.varlen_fwd(vd["q"], vd["k"], vd["v"], vd["g"], vd["beta"], vd["cu_seqlens"], vd["s0"], workspace=ws)

    _, vk_ms, vk_min = time_launches(vstep, max(10, args.steps // 2), args.warmup, torch)
    vbytes = chunk_alg_bytes(vspec.total * vspec.H, vspec.n_seq * vspec.H, 128, 128, 2, with_s0=True)
    return {"workload": name, "tokens": vspec.total, "longest": max(vspec.lengths), "kernel_ms": vk_ms,
            "kernel_ms_min": vk_min, "tokens_per_s": vspec.total / (vk_ms * 1e-3),
            "achieved": vbytes / (vk_ms * 1e-3) / 1e9, "unit": "GB/s", "alg_bytes_per_launch": vbytes}


def measure_prefill_1m(args, torch, kda, kda_inputs, device_inputs):
    """Million-token prefill, B=1, H=8, d=128, bf16 (long-memory gates): tokens/s of one call."""
    name = "prefill_b1_h8_t1m_d128_bf16"
    spec = kda_inputs.workload(name)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, batched=True)
    B, T, H, Dk, Dv = spec.n_seq, spec.lengths[0], spec.H, spec.Dk, spec.Dv
    ws = torch.empty(kda.chunk_workspace_bytes(B, T, H, Dk, Dv), dtype=torch.uint8, device="cuda")

    def pstep():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], workspace=ws)

    _, k_ms, k_min = time_launches(pstep, 5, max(1, args.warmup // 25), torch)
    alg = chunk_alg_bytes(B * T * H, B * H, Dk, Dv, 2, with_s0=False)
    return {"workload": name, "tokens": B * T, "kernel_ms": k_ms, "kernel_ms_min": k_min,
            "tokens_per_s": B * T / (k_ms * 1e-3), "achieved": alg / (k_ms * 1e-3) / 1e9, "unit": "GB/s",
            "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": alg,
            "workspace_bytes": ws.numel()}


def measure_raw_gates(args, torch, kda, kda_inputs, device_inputs):
    """The B=4 H=16 T=8192 batch fed raw: bf16 gate and beta logits, q and k not normalised; the
    kernels apply -softplus, the clamp, the logistic function and the L2 norm while loading."""
    name = "chunk_b4_h16_t8192_d128_bf16_raw_gates"
    base = kda_inputs.workload("chunk_b4_h16_t8192_d128_bf16")
    spec = kda_inputs.Spec(base.lengths, base.H, base.Dk, base.Dv, "bf16", "softplus", seed=base.seed,
                           g_logit=True, beta_logit=True, qk_l2norm=True, gate_dtype="bf16", name=name)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, batched=True)
    B, T, H, Dk, Dv = spec.n_seq, spec.lengths[0], spec.H, spec.Dk, spec.Dv
    ws = torch.empty(kda.chunk_workspace_bytes(B, T, H, Dk, Dv), dtype=torch.uint8, device="cuda")

    def rstep():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], workspace=ws, g_logit=True,
                      beta_logit=True, qk_l2norm=True)

    _, k_ms, k_min = time_launches(rstep, max(10, args.steps // 2), args.warmup, torch)
    alg = chunk_alg_bytes(B * T * H, B * H, Dk, Dv, 2, with_s0=False, gate_bytes=2)
    return {"workload": name, "tokens": B * T, "kernel_ms": k_ms, "kernel_ms_min": k_min,
            "tokens_per_s": B * T / (k_ms * 1e-3), "achieved": alg / (k_ms * 1e-3) / 1e9, "unit": "GB/s",
            "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": alg}


def measure_backward(args, torch, kda, kda_inputs, device_inputs):
    """Gradients of the B=4 H=16 T=8192 d=128 bf16 batch (seeded d_o, no final-state term)."""
    name = "chunk_b4_h16_t8192_d128_bf16"
    spec = kda_inputs.workload(name)
    inp = kda_inputs.generate(spec)
    d = device_inputs(inp, batched=True)
    B, T, H, Dk, Dv = spec.n_seq, spec.lengths[0], spec.H, spec.Dk, spec.Dv
    gen = torch.Generator(device="cuda").manual_seed(5)
    d_o = torch.randn((B, T, H, Dv), device="cuda", generator=gen)
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(B, T, H, Dk, Dv), dtype=torch.uint8, device="cuda")

    def bstep():
        kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, d["s0"], None, workspace=ws)

    _, k_ms, k_min = time_launches(bstep, max(5, args.steps // 5), max(2, args.warmup // 5), torch)
    # reads q, k, v (bf16), g, beta, d_o (fp32); writes dq, dk, dv, dg, dbeta (fp32) and ds0
    n_ht = B * T * H
    alg = n_ht * ((2 * Dk + Dv) * 2 + 4 * Dk + 4 + 4 * Dv + 4 * (3 * Dk + Dv) + 4) + B * H * Dk * Dv * 4
    return {"workload": name + "_backward", "tokens": B * T, "kernel_ms": k_ms, "kernel_ms_min": k_min,
            "tokens_per_s": B * T / (k_ms * 1e-3), "achieved": alg / (k_ms * 1e-3) / 1e9, "unit": "GB/s",
            "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": alg,
            "workspace_bytes": ws.numel(), "arith": "fp32 accumulation; split-bf16 three-pass products in the state recompute and column sums, fp32 MFMA elsewhere"}


if __name__ == "__main__":
    main()
