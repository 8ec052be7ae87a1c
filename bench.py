#!/usr/bin/env python3
"""Benchmark of the KDA / CKDA hot path on one MI355X.

One "step" is one chunkwise WY forward (kda_chunk_fwd) over the prefill batch
B=4, H=32, T=8192, d_k=d_v=128, bf16 inputs, fp32 state (the KDA workload,
seeded synthetic inputs already resident in HBM).  ``value`` is whole-job
prefill throughput in tokens/s (a token is one position across all H heads).
The same run also measures, outside the timed steps:
  * the CKDA prefill (same shape, gates in [-1, 1] and beta in [0, 2]);
  * the batched decode step (B=256, H=32, d=128, 64 consecutive steps on a
    512 MiB fp32 state), reported as state GB/s against the HBM peak;
  * the fp64 CPU oracle on a bounded sample of the prefill workload.

Prints ONE JSON line.  Timing: W untimed warm-up steps, then exactly K steps
between synchronisations, with HIP events recorded on the stream the kernel
is launched on (torch's current stream, which the binding launches on).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
PMC_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_kda_prefill_8k_counters.md")
KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_78_amd", "csrc", "kda_chunk.hip")


def chunk_bytes(B, T, H, dk, dv, es=2):
    """Algorithmic HBM bytes of one chunk-forward launch: q, k, alpha, v, beta read
    once, o written once, the fp32 start state read and the final state written."""
    per_head_token = es * (3 * dk + dv + 1) + es * dv
    return B * T * H * per_head_token + 2 * B * H * dk * dv * 4


def chunk_flops(B, T, H, dk, dv, C=64):
    """Algorithmic matrix flops of the chunk-WY forward per launch (per head-token:
    T, A, W, U, W S, Q S, A Delta, K^T Delta with the triangular halves counted once)."""
    per = 2 * (C // 2) * dk * 2 + 2 * (C // 2) * (dk + dv) + 2 * dk * dv * 3 + 2 * (C // 2) * dv
    return B * T * H * per


def decode_bytes(B, H, dk, dv, es=2):
    return 2 * B * H * dk * dv * 4 + B * H * (es * (3 * dk + dv + 1) + es * dv)


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by
    a copy-kernel calibration), if the counters were taken on the current kernel."""
    if not os.path.exists(PMC_FILE):
        return None
    txt = open(PMC_FILE).read()
    mh = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    mt = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not mh or not mt or mh.group(1) != kernel_hash():
        return None
    return float(mt.group(1))


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def bench_prefill(name, steps, warmup, log):
    import torch
    import gated_delta_rule_78_amd as kda
    from gated_delta_rule_78_amd.inputs import make_workload, WORKLOADS, to_torch
    w = WORKLOADS[name]
    t0 = time.time()
    inp = make_workload(name)
    q, k, v, a, b, s0 = to_torch(inp)
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = timed(lambda: kda.chunk_fwd(q, k, v, a, b, initial_state=s0, out=o, final_state=sT),
               steps, warmup, stream)
    del q, k, v, a, b, s0, o, sT
    torch.cuda.empty_cache()
    return w, ms, inp


def bench_decode(steps_rep, log):
    import torch
    import gated_delta_rule_78_amd as kda
    from gated_delta_rule_78_amd.inputs import make_workload, WORKLOADS, to_torch
    w = WORKLOADS["ckda_decode_b256"]
    t0 = time.time()
    inp = make_workload("ckda_decode_b256")
    q, k, v, a, b, s0 = to_torch(inp)
    log(f"[bench] decode: inputs ready in {time.time() - t0:.1f}s")
    S = s0.clone()
    o = torch.empty((w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    n = w.decode_steps
    times = []
    for rep in range(steps_rep + 1):
        S.copy_(s0)                      # restore the start state (not timed)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(n):
            kda.decode_step(q[t], k[t], v[t], a[t], b[t], S, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep > 0:                      # first repetition is the warm-up
            times.append(e0.elapsed_time(e1) / n)
    ms = float(np.median(times))
    return w, ms


def cpu_baseline(inp, budget_s, log):
    """The fp64 oracle on whole sequences of a sample of heads of the prefill
    workload; value scaled to the metric's unit (tokens/s across all H heads)."""
    import oracle
    m = inp.meta
    B, T, H = m["B"], m["T"], m["H"]
    cores = len(os.sched_getaffinity(0))
    cores = min(cores, 16)
    t0 = time.time()
    oracle.fwd(inp.q, inp.k, inp.v, inp.alpha, inp.beta, S0=inp.S0.reshape(B * H, m["dk"], m["dv"])[:1],
               heads=[0], col_block=max(1, m["dv"] // cores), nthreads=cores, want_o=True)
    one = time.time() - t0
    n = int(max(1, min(B * H, budget_s / max(one, 1e-3))))
    heads = list(range(n))
    t0 = time.time()
    oracle.fwd(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
               S0=inp.S0.reshape(B * H, m["dk"], m["dv"])[heads], heads=heads,
               col_block=max(1, (m["dv"] * n) // (4 * cores)) if n < 4 * cores else m["dv"],
               nthreads=cores, want_o=True)
    dt = time.time() - t0
    log(f"[bench] cpu oracle: {n} heads x T={T} in {dt:.1f}s on {cores} threads")
    head_tokens_per_s = n * T / dt
    return {"value": head_tokens_per_s / H, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {B * H} (b,h) heads of the B={B} H={H} T={T} d=128 KDA prefill, whole "
                      f"sequences, fp64, {dt:.1f}s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true", help="only the timed prefill steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the prefill shards over (b, h) with no exchange, which this single-GPU run does not exercise.",
              file=sys.stderr)
        sys.exit(2)
    log = lambda s: print(s, file=sys.stderr, flush=True)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import gated_delta_rule_78_amd as kda
    kda.lib()  # fail loudly if the HIP library is missing

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read, 1 GiB written")
        del src, dst

    w, ms, inp = bench_prefill("kda_prefill_8k", args.steps, args.warmup, log)
    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    nbytes = chunk_bytes(w.B, w.T, w.H, w.dk, w.dv)
    achieved = nbytes / (ms * 1e-3) / 1e9
    flops = chunk_flops(w.B, w.T, w.H, w.dk, w.dv)
    out = {
        "metric": "chunk-fwd tokens/s (H=32,d=128,T=8K bf16) + decode state GB/s, % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy; q,k L2-normalised N(0,1), v N(0,1), "
                "alpha=exp(-0.1 softplus(N)), beta=sigmoid(N), S0 N(0,0.02))",
        "config": {"workload": "kda_prefill_8k", "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "chunk": 64, "state": "fp32", "tokens_per_step": tokens},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(),
                     "kernel": "chunk_fwd_kernel<bf16,128,128>", "algorithmic_bytes_per_launch": nbytes,
                     "mfma_tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
                     "mfma_frac_algorithmic": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
    }
    log(f"[bench] kda prefill: {ms:.3f} ms/step, {value:.4g} tokens/s, {achieved:.1f} GB/s")
    if not args.no_extras:
        w3, ms3, _ = bench_prefill("ckda_prefill_8k", args.steps, args.warmup, log)
        out["ckda_prefill_8k"] = {"value": w3.B * w3.T / (ms3 * 1e-3), "unit": "tokens/s", "ms_per_step": ms3,
                                  "frac_hbm": chunk_bytes(w3.B, w3.T, w3.H, w3.dk, w3.dv) / (ms3 * 1e-3) / 1e9
                                  / HBM_PEAK_GBS}
        log(f"[bench] ckda prefill: {ms3:.3f} ms/step")
        wd, msd = bench_decode(3, log)
        db = decode_bytes(wd.B, wd.H, wd.dk, wd.dv)
        gbs = db / (msd * 1e-3) / 1e9
        out["decode"] = {"workload": "ckda_decode_b256", "B": wd.B, "H": wd.H, "dk": wd.dk, "dv": wd.dv,
                         "steps": wd.decode_steps, "ms_per_step": msd, "value": gbs, "unit": "GB/s",
                         "tokens_per_s": wd.B / (msd * 1e-3), "frac": gbs / HBM_PEAK_GBS,
                         "bytes_per_step": db}
        log(f"[bench] decode: {msd * 1e3:.1f} us/step, {gbs:.1f} GB/s")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
