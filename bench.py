"""Throughput benchmark of the gated delta-rule (KDA) forward pass on one MI355X.

Timed step: one kda_chunk_fwd call over the chunked-prefill batch B=4, H=16,
T=8192, d_k=d_v=128 (bf16 q/k/v, fp32 gates, fp32 state and output), inputs
and the workspace resident in HBM (the call launches the per-chunk preparation
kernel prep16_kernel and the state-chain kernel chain16_kernel).
value = B*T tokens per step / seconds per step, over the K timed steps.

Order of a default run: the calibration leg (plain HBM copy and matrix-core
loops), the other workloads, the flushed-cache protocol on the timed batch,
then the W warm-up and K timed steps.  The legs before the timed steps keep the
GPU busy for several seconds, so the timed steps run at a settled clock.

Also reported on the same JSON line:
  roofline      the call against HBM bandwidth: algorithmic bytes / mean launch time
                (events on the library's stream over the timed steps); bytes counted
                as 1,540 per head-token (o at 2 bytes) plus the final state, with the
                fp32-output byte count as a second, named figure; the flushed-cache
                median and min (512 MB written before each of 20 launches)
  mfma          the call's algorithmic FLOPs against the dense bf16 matrix-core peak,
                beside the ceiling that the HBM roofline puts on that fraction
  peaks         this GPU's plain-copy HBM rate and bf16 matrix-core rates, measured here
  fused         the single fused kernel (workspace NULL) on the same batch
  decode        single-token decode step, B=256, H=32, d=128: GB/s against HBM peak
  varlen        packed varlen prefill, 32 sequences, H=16, d=128
  prefill_1m    one million-token prefill, B=1, H=8, d=128
  raw_gates     the timed batch with bf16 gate/beta logits and the fused prologue
  backward      gradients of the timed batch
  cpu_baseline  the fp64 CPU oracle on the same chunked batch
  parity        max|err|/RMS of the timed output against that oracle run

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
                       [--only {chunk,decode,varlen,prefill_1m,raw_gates,backward,peaks}]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FLUSH_BYTES = 512 << 20         # written before each flushed-protocol launch (L2 + Infinity Cache are 256 MB)


def chunk_alg_bytes(n_head_tokens, n_heads, Dk, Dv, in_bytes, with_s0, gate_bytes=4, o_bytes=2):
    """Bytes the method must move once: q, k, v in the input type; g (Dk) and beta in the gate type;
    o (Dv, at o_bytes: 2 as the cost model counts it, 4 as the library writes it); the final state fp32
    (and the initial state when given)."""
    per_tok = (2 * Dk + Dv) * in_bytes + gate_bytes * (Dk + 1) + o_bytes * Dv
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


# Untimed calls before each measurement's warm-up, until the GPU clock has settled: its governor
# raises the clock over a few hundred milliseconds of sustained load (the B=4 H=16 call takes 0.55 ms
# at the first calls after idle and 0.47 ms once settled).
SETTLE_S = 0.3


def settle_clock(fn, torch, seconds=SETTLE_S):
    """Call fn, untimed, until `seconds` of wall time have passed; returns the number of calls."""
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_launches(fn, steps, warmup, torch, flush=None):
    """Run fn `warmup` times, then `steps` times bracketed by synchronize, on the current stream (the
    stream the library launches on).  Without `flush` the timed loop holds nothing but the calls: one
    event pair around all of them gives the mean launch time (events between calls cost the GPU about
    10 us each time), and a second, untimed pass with events around each call gives the median and
    min.  With `flush`, it runs before each launch, outside the per-call events of the timed loop.
    Returns wall seconds of the timed loop and the mean, median and min launch time in ms.  Before the
    warm-up, fn runs untimed until the clock has settled (settle_clock)."""
    settle_clock(fn, torch)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if flush is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mean = e0.elapsed_time(e1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t1 = time.perf_counter()
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    if flush is not None:
        wall, mean = time.perf_counter() - t1, float(per.mean())
    return wall, float(mean), float(np.median(per)), float(per.min())


def cpu_threads():
    """Threads for the CPU oracle: the CPUs this process may run on, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(env)) if env.isdigit() and int(env) > 0 else n


def measure_peaks(args, torch, kda):
    """This GPU's achievable rates: a plain copy of 1 GiB (2 GiB moved), median of 10; the two bf16
    matrix-core instructions on 8 workgroups of 4 waves per compute unit, median of 5."""
    st = torch.cuda.current_stream().cuda_stream
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)

    def copy():
        assert kda.calib_copy_raw(src.data_ptr(), dst.data_ptr(), nbytes, st) == 0

    _, c_mean, c_med, c_min = time_launches(copy, 10, 3, torch)
    out = {"copy": {"bytes_moved": 2 * nbytes, "median_ms": c_med, "min_ms": c_min,
                    "GB_s": 2 * nbytes / (c_med * 1e-3) / 1e9, "kernel": "kda_calib_copy (16-byte non-temporal)"}}
    del src, dst
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * n_cu
    buf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for kind, name, flops in [(0, "v_mfma_f32_16x16x32_bf16", 16 * 16 * 32 * 2),
                              (1, "v_mfma_f32_32x32x16_bf16", 32 * 32 * 16 * 2)]:
        iters = 20000 if kind == 0 else 10000

        def loop():
            assert kda.calib_mfma_raw(buf.data_ptr(), blocks, iters, kind, st) == 0

        _, m_mean, m_med, m_min = time_launches(loop, 5, 2, torch)
        total = blocks * 4 * 4 * iters * flops
        out[name] = {"median_ms": m_med, "TFLOP_s": total / (m_med * 1e-3) / 1e12,
                     "frac_of_peak": total / (m_med * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    out["compute_units"] = n_cu
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the calibration leg and the other workloads")
    ap.add_argument("--only", choices=["chunk", "decode", "varlen", "prefill_1m", "raw_gates", "backward", "peaks"],
                    default=None,
                    help="time one workload only (for profiler runs); prints its own JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run kda_calib_copy three times on MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path runs on a single device.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_65_amd as kda
    import kda_inputs
    from kda_inputs.device import device_inputs, to_dev

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kda.load_library()

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            assert kda.calib_copy_raw(src.data_ptr(), dst.data_ptr(), nbytes, st) == 0
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}))
        return

    solo = {"decode": lambda: measure_decode(args, torch, kda, kda_inputs, to_dev),
            "varlen": lambda: measure_varlen(args, torch, kda, kda_inputs, device_inputs),
            "prefill_1m": lambda: measure_prefill_1m(args, torch, kda, kda_inputs, device_inputs),
            "raw_gates": lambda: measure_raw_gates(args, torch, kda, kda_inputs, device_inputs),
            "backward": lambda: measure_backward(args, torch, kda, kda_inputs, device_inputs),
            "peaks": lambda: measure_peaks(args, torch, kda)}
    if args.only in solo:
        print(json.dumps({args.only: solo[args.only]()}))
        return
    extras = args.only is None and not args.no_extras

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

    tokens = B * T
    n_ht = tokens * H
    line_extras = {}
    flushed = None
    if extras:
        line_extras["peaks"] = measure_peaks(args, torch, kda)
        _, f_mean, f_med, f_min = time_launches(step_fused, 20, 3, torch)
        line_extras["fused"] = {"kernel": "chunk_fwd_kernel<128,false>", "kernel_ms": f_mean,
                                "kernel_ms_median": f_med, "kernel_ms_min": f_min,
                                "tokens_per_s": tokens / (f_mean * 1e-3)}
        line_extras["decode"] = solo["decode"]()
        line_extras["varlen"] = solo["varlen"]()
        line_extras["prefill_1m"] = solo["prefill_1m"]()
        line_extras["raw_gates"] = solo["raw_gates"]()
        line_extras["backward"] = solo["backward"]()
        # the cost model's protocol: 512 MB written before each of 20 launches, median and min
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        _, fl_mean, fl_med, fl_min = time_launches(step, 20, 3, torch, flush=lambda: scratch.fill_(1.0))
        flushed = {"median_ms": fl_med, "min_ms": fl_min, "flush_bytes": FLUSH_BYTES}
        del scratch

    wall, k_mean, k_med, k_min = time_launches(step, args.steps, args.warmup, torch)
    ms_per_step = wall * 1e3 / args.steps
    value = tokens * args.steps / wall
    alg_bytes = chunk_alg_bytes(n_ht, B * H, Dk, Dv, 2, with_s0=False)            # o counted at 2 bytes
    alg_bytes_o32 = chunk_alg_bytes(n_ht, B * H, Dk, Dv, 2, with_s0=False, o_bytes=4)
    alg_flops = chunk_alg_flops(n_ht, Dk, Dv)
    gbs = alg_bytes / (k_mean * 1e-3) / 1e9
    tflops = alg_flops / (k_mean * 1e-3) / 1e12
    # at the HBM roofline the call takes alg_bytes / peak; the matrix-core fraction cannot exceed
    # what that time allows
    mfma_ceiling = alg_flops / (alg_bytes / (HBM_PEAK_GBS * 1e9)) / 1e12 / BF16_MFMA_PEAK_TFLOPS

    roofline = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(name),
                "kernel": "prep16_kernel<128,false> + chain16_kernel<128,false> (one kda_chunk_fwd call)",
                "kernel_ms": k_mean, "kernel_ms_median": k_med, "kernel_ms_min": k_min,
                "alg_bytes_per_launch": alg_bytes,
                "alg_bytes_def": "1540 B per head-token (q,k,v bf16 768; g fp32 512; beta 4; o 256 at 2 B) "
                                 "+ final state fp32",
                "fp32_o": {"alg_bytes_per_launch": alg_bytes_o32,
                           "achieved": alg_bytes_o32 / (k_mean * 1e-3) / 1e9,
                           "frac": alg_bytes_o32 / (k_mean * 1e-3) / 1e9 / HBM_PEAK_GBS},
                "workspace_bytes": ws.numel()}
    if flushed is not None:
        flushed["frac_median"] = alg_bytes / (flushed["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        roofline["flushed"] = flushed
    if "peaks" in line_extras:
        roofline["frac_of_copy_rate"] = gbs / line_extras["peaks"]["copy"]["GB_s"]

    line = {
        "metric": "KDA fwd tokens/s (H=16,d=128,T=8192) + % MFMA peak; decode % HBM BW",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": SETTLE_S,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "T": T, "H": H, "d_k": Dk, "d_v": Dv, "chunk": 64,
                   "qkv": "bf16", "gates": "fp32", "state": "fp32", "output": "fp32", "parallelism": "none"},
        "roofline": roofline,
        "mfma": {"achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "alg_flops_per_launch": alg_flops,
                 "ceiling_frac_at_hbm_roofline": mfma_ceiling},
    }
    line.update(line_extras)

    if args.only is None and not args.no_cpu_baseline:
        import oracle
        nthreads = cpu_threads()
        t0 = time.perf_counter()
        o_ref, s_ref = oracle.forward_inputs(inp, nthreads=nthreads)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": tokens / dt, "unit": "tokens/s", "cores": nthreads,
                                "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle", "seconds": dt,
                                "sample": f"the whole timed batch ({B}x{T} tokens, {H} heads, all {Dv} columns), "
                                          "fp64 token-by-token recurrence"}
        o_gpu = out["o"].reshape(tokens, H, Dv).cpu().numpy()
        line["parity"] = {"o_err": oracle.rel_err(o_gpu, o_ref), "s_err": oracle.rel_err(out["s"].cpu().numpy(), s_ref),
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

    _, dk_ms, dk_med, dk_min = time_launches(dstep, max(20, args.steps), args.warmup, torch)
    dbytes = decode_alg_bytes(Bd, Hd, 128, 128, 2)
    dgbs = dbytes / (dk_ms * 1e-3) / 1e9
    return {"workload": name, "kernel_ms": dk_ms, "kernel_ms_median": dk_med, "kernel_ms_min": dk_min, "achieved": dgbs,
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

    _, vk_ms, vk_med, vk_min = time_launches(vstep, max(10, args.steps // 2), args.warmup, torch)
    vbytes = chunk_alg_bytes(vspec.total * vspec.H, vspec.n_seq * vspec.H, 128, 128, 2, with_s0=True)
    return {"workload": name, "tokens": vspec.total, "longest": max(vspec.lengths), "kernel_ms": vk_ms,
            "kernel_ms_median": vk_med, "kernel_ms_min": vk_min, "tokens_per_s": vspec.total / (vk_ms * 1e-3),
            "achieved": vbytes / (vk_ms * 1e-3) / 1e9, "unit": "GB/s",
            "frac": vbytes / (vk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": vbytes}


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

    _, k_ms, k_med, k_min = time_launches(pstep, 5, max(1, args.warmup // 25), torch)
    alg = chunk_alg_bytes(B * T * H, B * H, Dk, Dv, 2, with_s0=False)
    return {"workload": name, "tokens": B * T, "kernel_ms": k_ms, "kernel_ms_median": k_med, "kernel_ms_min": k_min,
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

    _, k_ms, k_med, k_min = time_launches(rstep, max(10, args.steps // 2), args.warmup, torch)
    alg = chunk_alg_bytes(B * T * H, B * H, Dk, Dv, 2, with_s0=False, gate_bytes=2)
    return {"workload": name, "tokens": B * T, "kernel_ms": k_ms, "kernel_ms_median": k_med, "kernel_ms_min": k_min,
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

    _, k_ms, k_med, k_min = time_launches(bstep, max(5, args.steps // 5), max(2, args.warmup // 5), torch)
    # reads q, k, v (bf16), g, beta, d_o (fp32); writes dq, dk, dv, dg, dbeta (fp32) and ds0
    n_ht = B * T * H
    alg = n_ht * ((2 * Dk + Dv) * 2 + 4 * Dk + 4 + 4 * Dv + 4 * (3 * Dk + Dv) + 4) + B * H * Dk * Dv * 4
    return {"workload": name + "_backward", "tokens": B * T, "kernel_ms": k_ms, "kernel_ms_median": k_med,
            "kernel_ms_min": k_min,
            "tokens_per_s": B * T / (k_ms * 1e-3), "achieved": alg / (k_ms * 1e-3) / 1e9, "unit": "GB/s",
            "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": alg,
            "workspace_bytes": ws.numel(), "traffic": measured_traffic(name + "_backward"), "arith": "fp32 accumulation; split-bf16 three-pass products in the state recompute, the reverse chain, the column sums and the decayed Gram contractions, fp32 MFMA through the inverse"}


if __name__ == "__main__":
    main()
