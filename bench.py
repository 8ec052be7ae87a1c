#!/usr/bin/env python3
"""Benchmark of the KDA / CKDA hot path on one MI355X.

One "step" is one chunkwise WY forward over the prefill batch B=4, H=32,
T=8192, d_k=d_v=128, bf16 inputs, fp32 state (the KDA workload, seeded
synthetic inputs already resident in HBM), through the path the library picks
for the shape (``pick_path``: the two-pass forward here, i.e. kda_chunk_records
then kda_chunk_apply_records on a preallocated workspace).  ``value`` is
whole-job prefill throughput in tokens/s (a token is one position across all H
heads).  The same run also measures, outside the timed steps:
  * the CKDA prefill (same shape, gates in [-1, 1] and beta in [0, 2]);
  * the long-context CKDA prefill (B=1, H=16, T=131072);
  * the Gated DeltaNet-2 prefill (decoupled erase / write gates, B=4, H=32, T=8192);
  * the batched decode step (B=256, H=32, d=128, 64 consecutive steps on a
    512 MiB fp32 state), reported as state GB/s against the HBM peak;
  * the fp64 CPU oracle on a bounded sample of the prefill workload.

Prints ONE JSON line.  Timing: W untimed warm-up steps, then exactly K steps
between synchronisations, with HIP events recorded on the stream the kernels
are launched on (torch's current stream, which the binding passes to the
library); an event between the two launches of a step gives each kernel's own
average duration for the roofline entry.
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
MFMA_FP32_PEAK_TFLOPS = 157.3   # dense fp32 matrix cores
CSRC = os.path.join(ROOT, "gated_delta_rule_78_amd", "csrc")
# the rocprofv3 counter summary of each kernel, and the sources that kernel is built from
PMC_FILES = {
    "chunk_records": (os.path.join(ROOT, "profiles", "chunk_records_kda_prefill_8k_counters.md"),
                      ["kda_records.hip", "kda_tile.h", "kda_record.h", "kda_common.h"]),
    "chunk_state": (os.path.join(ROOT, "profiles", "chunk_state_kda_prefill_8k_counters.md"),
                    ["kda_walk.hip", "kda_tile.h", "kda_record.h", "kda_common.h"]),
    "chunk_fused": (os.path.join(ROOT, "profiles", "chunk_fused_kda_prefill_8k_counters.md"),
                    ["kda_chunk.hip", "kda_tile.h", "kda_common.h"]),
    "decode": (os.path.join(ROOT, "profiles", "decode_ckda_decode_b256_counters.md"),
               ["kda_decode.hip", "kda_common.h"]),
}
# the bf16 walk record of one (b, h, chunk): A, M~ hi and M~ lo, three lower 64 x 64 bf16
# matrices stored as row-major blocks (rows 0..31 x 32 columns, rows 32..63 x 64 columns;
# the image the state pass moves into LDS as it is)
RECORD_BYTES = {128: 18432, 64: 18432}


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


def records_bytes(B, T, H, dk, es=2):
    """Own bytes of one kda_chunk_records launch: q, k, alpha, beta read once, one record
    per (b, h, chunk) written."""
    nch = (T + 63) // 64
    return B * T * H * es * (3 * dk + 1) + B * H * nch * RECORD_BYTES[dk]


def state_bytes(B, T, H, dk, dv, es=2):
    """Own bytes of one kda_chunk_apply_records launch: every record read once, q, k,
    alpha, v read and o written once, start state read and final state written."""
    nch = (T + 63) // 64
    return (B * H * nch * RECORD_BYTES[dk] + B * T * H * es * (3 * dk + 2 * dv)
            + 2 * B * H * dk * dv * 4)


def decode_bytes(B, H, dk, dv, es=2, tokens=1):
    """Algorithmic bytes of one decode call: the fp32 state read and written once, and
    per token q, k, alpha, v, beta read and o written."""
    return 2 * B * H * dk * dv * 4 + tokens * B * H * (es * (3 * dk + dv + 1) + es * dv)


def kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by
    a copy-kernel calibration), if the counters were taken on the current sources."""
    path, files = PMC_FILES[kernel]
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    mh = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    mt = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not mh or not mt or mh.group(1) != kernel_hash(files):
        return None
    return float(mt.group(1))


UTIL_FILES = {  # rocprofv3 MfmaUtil / VALUBusy summaries, per kernel key
    "chunk_records": os.path.join(ROOT, "profiles", "utilisation_kda_prefill_8k.md"),
    "chunk_state": os.path.join(ROOT, "profiles", "utilisation_kda_prefill_8k.md"),
    "decode": os.path.join(ROOT, "profiles", "utilisation_ckda_decode_b256.md"),
    "bwd_records": os.path.join(ROOT, "profiles", "utilisation_ckda_backward_8k.md"),
    "bwd_state": os.path.join(ROOT, "profiles", "utilisation_ckda_backward_8k.md"),
    "bwd_adjoint": os.path.join(ROOT, "profiles", "utilisation_ckda_backward_8k.md"),
    "bwd_grads": os.path.join(ROOT, "profiles", "utilisation_ckda_backward_8k.md"),
}
UTIL_SOURCES = {"bwd_records": ["kda_bwd.hip", "kda_internal.h", "kda_common.h"]}
for _k in ("bwd_state", "bwd_adjoint", "bwd_grads"):
    UTIL_SOURCES[_k] = UTIL_SOURCES["bwd_records"]


def stored_util(kernel):
    """rocprofv3 matrix-core and VALU busy percentages of `kernel` ({"mfma_busy_pct",
    "valu_busy_pct"}), if the counters were taken on the current sources; else None."""
    path = UTIL_FILES.get(kernel)
    if not path or not os.path.exists(path):
        return None
    files = UTIL_SOURCES.get(kernel) or PMC_FILES[kernel][1]
    m = re.search(r"^- %s: mfma_busy_pct=([0-9.]+) valu_busy_pct=([0-9.]+) kernel_source_sha256_16=([0-9a-f]+)"
                  % re.escape(kernel), open(path).read(), re.M)
    if not m or m.group(3) != kernel_hash(files):
        return None
    return {"mfma_busy_pct": float(m.group(1)), "valu_busy_pct": float(m.group(2))}


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


def timed_split(first, second, steps, warmup, stream):
    """K steps of first(); second(), events around each launch.  Returns (ms per step,
    mean ms of first, mean ms of second)."""
    import torch
    for _ in range(warmup):
        first()
        second()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    for i in range(steps):
        ev[2 * i].record(stream)
        first()
        ev[2 * i + 1].record(stream)
        second()
    ev[2 * steps].record(stream)
    torch.cuda.synchronize()
    t1 = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
    t2 = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(steps)) / steps
    return ev[0].elapsed_time(ev[2 * steps]) / steps, t1, t2


def bench_prefill(name, steps, warmup, log):
    """Times the chunk forward of workload `name` on the path the library picks.
    Returns (workload, result dict, host inputs)."""
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
    path = kda.pick_path(w.B, w.T, w.H, w.dk, w.dv)
    res = {"path": path}
    if w.gates == "gdn2":
        # Gated DeltaNet-2: erase / write gates in place of beta, two-pass path
        def dev(x):
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        e, wg = dev(inp.erase), dev(inp.write)
        ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
        ms = timed(lambda: kda.gdn2_chunk_fwd(q, k, v, a, e, wg, initial_state=s0, out=o, final_state=sT,
                                              workspace=ws), steps, warmup, stream)
        res.update(path="gdn2-twopass", ms=ms, kernels={"gdn2_chunk_fwd": ms})
        del ws, e, wg
    elif w.gates == "sfda":
        # SFDA: complex rotation-decay gates in alpha's place, two-pass path
        ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
        ms = timed(lambda: kda.sfda_chunk_fwd(q, k, v, a, b, initial_state=s0, out=o, final_state=sT,
                                              workspace=ws), steps, warmup, stream)
        res.update(path="sfda-twopass", ms=ms, kernels={"sfda_chunk_fwd": ms})
        del ws
    elif path == "twopass":
        ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
        ms, t1, t2 = timed_split(lambda: kda.chunk_records(q, k, a, b, workspace=ws, dv=w.dv),
                                 lambda: kda.chunk_apply_records(ws, q, k, a, v, s0, out=o, final_state=sT),
                                 steps, warmup, stream)
        res.update(ms=ms, kernels={"chunk_records": t1, "chunk_state": t2},
                   workspace_bytes=ws.numel())
        del ws
    else:
        ms = timed(lambda: kda.chunk_fwd(q, k, v, a, b, initial_state=s0, out=o, final_state=sT, path="fused"),
                   steps, warmup, stream)
        res.update(ms=ms, kernels={"chunk_fused": ms})
    del q, k, v, a, b, s0, o, sT
    torch.cuda.empty_cache()
    return w, res, inp


def bwd_flops(B, T, H, dk, dv, C=64):
    """Dense product flops of the chunk backward per call (forward recomputed inside): per
    chunk A, D, W (records); Delta, S' (forward walk); dDelta, dS (adjoint walk); dQg, dKr,
    dW, dA, dV, dMt, dKg, dMt Mt^T, M^T X and the block-anchored products (gradients)."""
    nch = B * H * ((T + C - 1) // C)
    mm = lambda m, n, k: 2 * m * n * k
    anchored = sum(mm(C - s, dk, s) for s in (16, 32, 48))        # PA (or PD) over the three blocks
    per = (mm(C, C, dk) * 2 + mm(C, dk, C)                           # A, D, W
           + mm(C, dv, C + dk) + mm(dk, dv, C)                       # Delta, S'
           + mm(C, dv, dk + C) + mm(dk, dv, 2 * C)                   # dDelta, dS
           + 3 * mm(C, dk, dv) + mm(C, C, dv) + mm(C, dv, C)         # dQg, dKr, dW, dA, dV
           + mm(C, C, dv + dk) + mm(C, dk, C) + 2 * mm(C, C, C)      # dMt, dKg, X, dT
           + 2 * anchored + sum(mm(16, dk, 2 * n) for n in (48, 32, 16)))  # PA, PD, F
    return nch * per


def bench_backward(steps, warmup, log, name="ckda_prefill_8k"):
    """Times kda_chunk_bwd (kda_gdn2_chunk_bwd, kda_sfda_chunk_bwd for those gates) on workload `name`
    (start state and a final-state gradient given).  Returns (workload, ms per call)."""
    import torch
    import gated_delta_rule_78_amd as kda
    from gated_delta_rule_78_amd.inputs import make_workload, make_upstream, WORKLOADS, to_torch
    w = WORKLOADS[name]
    t0 = time.time()
    inp = make_workload(name)
    q, k, v, a, b, s0 = to_torch(inp)
    dO, dST = make_upstream(w.B, w.T, w.H, w.dk, w.dv, w.dtype, seed=90)
    d_o = torch.from_numpy(np.ascontiguousarray(dO).view(np.int16)).to("cuda").view(torch.bfloat16)
    dst = torch.from_numpy(dST).to("cuda")
    ws = torch.empty(kda.bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
    log(f"[bench] {name} backward: inputs ready in {time.time() - t0:.1f}s, workspace {ws.numel() / 1e9:.2f} GB")
    stream = torch.cuda.current_stream()
    if w.gates == "gdn2":
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        e, g = up(inp.erase), up(inp.write)
        call = lambda: kda.gdn2_chunk_bwd(q, k, v, a, e, g, d_o, initial_state=s0, d_final_state=dst, workspace=ws)
    elif w.gates == "sfda":
        call = lambda: kda.sfda_chunk_bwd(q, k, v, a, b, d_o, initial_state=s0, d_final_state=dst, workspace=ws)
    else:
        call = lambda: kda.chunk_bwd(q, k, v, a, b, d_o, initial_state=s0, d_final_state=dst, workspace=ws)
    ms = timed(call, steps, warmup, stream)
    del q, k, v, a, b, s0, d_o, dst, ws, call
    torch.cuda.empty_cache()
    return w, ms


def kernel_bytes(kernel, w):
    if kernel == "chunk_records":
        return records_bytes(w.B, w.T, w.H, w.dk)
    if kernel == "chunk_state":
        return state_bytes(w.B, w.T, w.H, w.dk, w.dv)
    return chunk_bytes(w.B, w.T, w.H, w.dk, w.dv)


def bench_decode(steps_rep, log, name="ckda_decode_b256"):
    import torch
    import gated_delta_rule_78_amd as kda
    from gated_delta_rule_78_amd.inputs import make_workload, WORKLOADS, to_torch
    w = WORKLOADS[name]
    step = kda.sfda_decode_step if w.gates == "sfda" else kda.decode_step
    t0 = time.time()
    inp = make_workload(name)
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
            step(q[t], k[t], v[t], a[t], b[t], S, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep > 0:                      # first repetition is the warm-up
            times.append(e0.elapsed_time(e1) / n)
    ms = float(np.median(times))
    return w, ms


def bench_decode_tokens(ntok, log, reps=3):
    """The decode workload's 64 tokens as 64 / ntok calls of ntok tokens each (the state
    read and written once per call)."""
    import torch
    import gated_delta_rule_78_amd as kda
    from gated_delta_rule_78_amd.inputs import make_workload, WORKLOADS, to_torch
    w = WORKLOADS["ckda_decode_b256"]
    inp = make_workload("ckda_decode_b256")
    q, k, v, a, b, s0 = to_torch(inp)
    # [steps, B, H, .] -> calls of [B, ntok, H, .]
    calls = []
    for c in range(w.decode_steps // ntok):
        sl = slice(c * ntok, (c + 1) * ntok)
        calls.append(tuple(x[sl].transpose(0, 1).contiguous() for x in (q, k, v, a, b)))
    S = s0.clone()
    o = torch.empty((w.B, ntok, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for rep in range(reps + 1):
        S.copy_(s0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for cq, ck, cv, ca, cb in calls:
            kda.decode_tokens(cq, ck, cv, ca, cb, S, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep > 0:
            times.append(e0.elapsed_time(e1) / len(calls))
    return w, float(np.median(times)), ntok


def host_cpus():
    """(threads to use, description): the CPUs this process may run on, bounded by the
    cgroup CPU quota where one is set (more threads than the quota only time-slice)."""
    n = len(os.sched_getaffinity(0))
    note = f"{n} CPUs in the affinity mask"
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            lim = max(1, int(-(-int(quota) // int(period))))
            note += f", cgroup quota {int(quota) / int(period):g} CPUs"
            n = min(n, lim)
    except (OSError, ValueError):
        pass
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, f"{model}; {note}"


def cpu_baseline(inp, budget_s, log):
    """The fp64 oracle on whole sequences of a sample of heads of the prefill
    workload, on every CPU this process may use; value scaled to the metric's unit
    (tokens/s across all H heads)."""
    import oracle
    m = inp.meta
    B, T, H = m["B"], m["T"], m["H"]
    cores, cpu = host_cpus()
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
    log(f"[bench] cpu oracle: {n} heads x T={T} in {dt:.1f}s on {cores} threads ({cpu})")
    head_tokens_per_s = n * T / dt
    return {"value": head_tokens_per_s / H, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu": cpu,
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
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode measurement (for profiling the decode kernel)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="only the backward measurement (for profiling the backward kernels)")
    ap.add_argument("--prefill", default=None,
                    choices=("kda_prefill_8k", "ckda_prefill_8k", "ckda_prefill_128k", "gdn2_prefill_8k",
                             "sfda_prefill_8k"),
                    help="only this prefill workload (for profiling its kernels); prints its own line")
    ap.add_argument("--bwd-workload", default="ckda_prefill_8k",
                    choices=("ckda_prefill_8k", "gdn2_prefill_8k", "sfda_prefill_8k", "ckda_prefill_128k"),
                    help="workload of --bwd-only")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
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

    if args.decode_only:
        wd, msd = bench_decode(max(1, args.steps // 10), log)
        db = decode_bytes(wd.B, wd.H, wd.dk, wd.dv)
        gbs = db / (msd * 1e-3) / 1e9
        print(json.dumps({"workload": "ckda_decode_b256", "ms_per_step": msd, "value": gbs, "unit": "GB/s",
                          "frac": gbs / HBM_PEAK_GBS, "bytes_per_step": db}), flush=True)
        return
    if args.prefill:
        wp, rp, _ = bench_prefill(args.prefill, args.steps, args.warmup, log)
        print(json.dumps({"workload": args.prefill, "path": rp["path"], "ms_per_step": rp["ms"],
                          "tokens_per_s": wp.B * wp.T / (rp["ms"] * 1e-3), "kernels_ms": rp["kernels"]}), flush=True)
        return
    if args.bwd_only:
        wb, msb = bench_backward(max(1, args.steps // 4), 1, log, name=args.bwd_workload)
        fl = bwd_flops(wb.B, wb.T, wb.H, wb.dk, wb.dv)
        print(json.dumps({"workload": f"{wb.name} backward", "ms_per_call": msb,
                          "tokens_per_s": wb.B * wb.T / (msb * 1e-3),
                          "tflops_fp32": fl / (msb * 1e-3) / 1e12}), flush=True)
        return
    w, res, inp = bench_prefill("kda_prefill_8k", args.steps, args.warmup, log)
    ms = res["ms"]
    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    nbytes = chunk_bytes(w.B, w.T, w.H, w.dk, w.dv)
    path_gbs = nbytes / (ms * 1e-3) / 1e9
    flops = chunk_flops(w.B, w.T, w.H, w.dk, w.dv)
    # roofline of the dominant kernel: the path's algorithmic bytes per launch (each launch
    # of the path covers all B*T*H head-tokens: 1,282 B each plus the two states) over that
    # kernel's own mean duration; beside it the whole path against the same floor
    dom = max(res["kernels"], key=res["kernels"].get)
    dom_ms = res["kernels"][dom]
    achieved = nbytes / (dom_ms * 1e-3) / 1e9
    roof_tokens_per_s = tokens / (nbytes / (HBM_PEAK_GBS * 1e9))
    own = {k2: {"ms": t2, "own_bytes": kernel_bytes(k2, w), "own_gbs": kernel_bytes(k2, w) / (t2 * 1e-3) / 1e9}
           for k2, t2 in res["kernels"].items()}
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
                   "chunk": 64, "state": "fp32", "tokens_per_step": tokens, "path": res["path"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(dom),
                     "kernel": dom, "kernel_ms": dom_ms, "algorithmic_bytes_per_launch": nbytes,
                     "algorithmic_bytes_per_head_token": chunk_bytes(1, 1, 1, w.dk, w.dv) - 2 * w.dk * w.dv * 4,
                     "path_frac": value / roof_tokens_per_s, "path_roofline_tokens_per_s": roof_tokens_per_s,
                     "path_ms": ms, "kernel_own_traffic": own,
                     "rocprof_busy": {k2: stored_util(k2) for k2 in res["kernels"] if k2 in UTIL_FILES},
                     "mfma": {"tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
                              "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}},
    }
    log(f"[bench] kda prefill ({res['path']}): {ms:.3f} ms/step, {value:.4g} tokens/s; "
        + ", ".join(f"{k2} {v2:.3f} ms" for k2, v2 in res["kernels"].items()))
    if not args.no_extras:
        for name, steps in (("ckda_prefill_8k", args.steps), ("ckda_prefill_128k", max(2, args.steps // 4)),
                            ("gdn2_prefill_8k", args.steps), ("sfda_prefill_8k", args.steps)):
            w3, r3, _ = bench_prefill(name, steps, min(args.warmup, 2), log)
            ms3 = r3["ms"]
            out[name] = {"value": w3.B * w3.T / (ms3 * 1e-3), "unit": "tokens/s", "ms_per_step": ms3,
                         "steps": steps, "path": r3["path"], "kernels_ms": r3["kernels"],
                         "frac_hbm": chunk_bytes(w3.B, w3.T, w3.H, w3.dk, w3.dv) / (ms3 * 1e-3) / 1e9
                         / HBM_PEAK_GBS}
            log(f"[bench] {name} ({r3['path']}): {ms3:.3f} ms/step")
        wd, msd = bench_decode(3, log)
        db = decode_bytes(wd.B, wd.H, wd.dk, wd.dv)
        gbs = db / (msd * 1e-3) / 1e9
        out["decode"] = {"workload": "ckda_decode_b256", "B": wd.B, "H": wd.H, "dk": wd.dk, "dv": wd.dv,
                         "steps": wd.decode_steps, "ms_per_step": msd, "value": gbs, "unit": "GB/s",
                         "tokens_per_s": wd.B / (msd * 1e-3), "frac": gbs / HBM_PEAK_GBS,
                         "bytes_per_step": db, "traffic": stored_traffic("decode"),
                         "rocprof_busy": stored_util("decode")}
        log(f"[bench] decode: {msd * 1e3:.1f} us/step, {gbs:.1f} GB/s")
        ws_, mss = bench_decode(3, log, name="sfda_decode_b256")
        gbs_s = db / (mss * 1e-3) / 1e9
        out["sfda_decode"] = {"workload": "sfda_decode_b256", "ms_per_step": mss, "value": gbs_s, "unit": "GB/s",
                              "tokens_per_s": ws_.B / (mss * 1e-3), "frac": gbs_s / HBM_PEAK_GBS}
        log(f"[bench] sfda decode: {mss * 1e3:.1f} us/step, {gbs_s:.1f} GB/s")
        wb, msb = bench_backward(max(2, args.steps // 4), 1, log)
        flb = bwd_flops(wb.B, wb.T, wb.H, wb.dk, wb.dv)
        out["ckda_backward_8k"] = {"workload": "ckda_prefill_8k", "ms_per_call": msb,
                                   "tokens_per_s": wb.B * wb.T / (msb * 1e-3), "dtype": "f32",
                                   "dense_flops_per_call": flb, "tflops_fp32": flb / (msb * 1e-3) / 1e12,
                                   "frac_fp32_mfma": flb / (msb * 1e-3) / 1e12 / MFMA_FP32_PEAK_TFLOPS,
                                   "rocprof_busy": {k2: stored_util(k2) for k2 in
                                                    ("bwd_records", "bwd_state", "bwd_adjoint", "bwd_grads")}}
        log(f"[bench] ckda backward 8k: {msb:.3f} ms/call, {flb / (msb * 1e-3) / 1e12:.1f} dense fp32 TFLOP/s")
        wg, msg = bench_backward(max(2, args.steps // 4), 1, log, name="gdn2_prefill_8k")
        out["gdn2_backward_8k"] = {"workload": "gdn2_prefill_8k", "ms_per_call": msg,
                                   "tokens_per_s": wg.B * wg.T / (msg * 1e-3), "dtype": "f32"}
        log(f"[bench] gdn2 backward 8k: {msg:.3f} ms/call")
        wsf, mss_ = bench_backward(max(2, args.steps // 4), 1, log, name="sfda_prefill_8k")
        out["sfda_backward_8k"] = {"workload": "sfda_prefill_8k", "ms_per_call": mss_,
                                   "tokens_per_s": wsf.B * wsf.T / (mss_ * 1e-3), "dtype": "f32"}
        log(f"[bench] sfda backward 8k: {mss_:.3f} ms/call")
        wt, mst, ntk = bench_decode_tokens(4, log)
        bt_ = decode_bytes(wt.B, wt.H, wt.dk, wt.dv, tokens=ntk)
        out["decode_tokens"] = {"workload": "ckda_decode_b256", "tokens_per_call": ntk, "ms_per_call": mst,
                                "us_per_token": mst * 1e3 / ntk, "tokens_per_s": wt.B * ntk / (mst * 1e-3),
                                "value": bt_ / (mst * 1e-3) / 1e9, "unit": "GB/s",
                                "frac": bt_ / (mst * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] decode, {ntk} tokens per call: {mst * 1e3:.1f} us/call ({mst * 1e3 / ntk:.1f} us/token)")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
