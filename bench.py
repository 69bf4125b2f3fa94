#!/usr/bin/env python3
"""Throughput of the W4 verify projection + greedy verify on one MI355X.

One step is the whole hot path over one verify block: the W4 group-64 QMM
y[M,N] = x[M,K] . W^T (vqv_qgemm), then the per-row argmax and accept walk
over y (vqv_verify). The default workload is the target projection M=8,
K=5120, N=17408 with bf16 activations and a verify block of T=8. Inputs are
seeded synthetic tensors of that shape, resident in HBM before timing. The
weights rotate through enough copies that every step streams them from HBM
rather than from the 256 MB Infinity Cache.

Prints one JSON line. `value` is verified rows per second (M rows per step);
`roofline` reports the QMM kernel's algorithmic bytes per launch divided by
its mean launch time (HIP events around each launch on the launch stream)
against the 8 TB/s HBM peak; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verified rows/s + achieved HBM GB/s, W4 M=8 QMM K=5120 N=17408"
MALL_BYTES = 256 << 20

# workload -> (verify block T, sequences B) for the steps that include verify
VERIFY = {"tiny": (8, 1), "target": (8, 1), "vocab_verify": (8, 1), "batched_vocab": (16, 4)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def qgemm_bytes(M, K, N, esz):
    return K * N // 2 + 4 * N * (K // 64) + M * K * esz + 4 * M * N


def traffic_record(workload, M):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs,
    valid only while the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", "qgemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "w4_gemm_vqv_amd", "csrc", "qgemm.hip"), "rb").read()
    entry = rec.get("workloads", {}).get(f"{workload}:M={M}")
    if not entry or rec.get("qgemm_hip_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return entry["fetch_bytes"] + entry["write_bytes"]


def cpu_baseline(c, M, T, B, budget_s):
    """The oracle, untuned, on a column sample of the same workload, scaled to
    rows/s of the full problem."""
    import numpy as np
    from oracle import qgemm_ref, verify_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the process's CPU share
        threads = len(os.sched_getaffinity(0))
    N = c["N"]
    x = c["x"][:M]

    def run(ncols):
        t0 = time.perf_counter()
        qgemm_ref(x, c["act"], c["wq"][:ncols], c["scales"][:ncols], c["biases"][:ncols])
        return time.perf_counter() - t0

    probe = min(N, 1024)
    t_probe = run(probe)
    ncols = int(min(N, max(probe, probe * (budget_s / 3) / max(t_probe, 1e-6))))
    times = [run(ncols) for _ in range(3)]
    t_q = statistics.median(times) * N / ncols
    t_v = 0.0
    if T:
        rng = np.random.default_rng(0)
        lg = rng.standard_normal((B * T, N)).astype(np.float32)
        d = rng.integers(0, N, size=(B, T - 1)).astype(np.int32)
        t0 = time.perf_counter()
        verify_ref(lg, d, B, T)
        t_v = time.perf_counter() - t0
    return {"value": M / (t_q + t_v), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"qgemm over {ncols} of {N} columns (median of 3, scaled to N) + "
                      f"verify over all {B * T} x {N} logits; host cpus {os.cpu_count()}",
            "seconds_per_step": t_q + t_v}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="target",
                    choices=["tiny", "target", "draft_w4a32", "vocab_verify", "batched_vocab",
                             "gate_up"])
    ap.add_argument("--m", type=int, default=None, help="rows (default: the workload's M)")
    ap.add_argument("--rotate", type=int, default=None, help="weight copies cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py measures one GPU only: this build has no multi-GPU path "
                  f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import w4_gemm_vqv_amd as vqv

    vqv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = gen.make_config(args.workload)
    M = args.m or c["M"]
    K, N, act = c["K"], c["N"], c["act"]
    esz = 4 if act == "fp32" else 2
    T, B = VERIFY.get(args.workload, (0, 0))
    if T:
        if B == 1:
            T = M
        elif B * T != M:
            raise SystemExit(f"{args.workload}: M must be {B * T}")

    wbytes = K * N // 2 + 4 * N * (K // 64)
    R = args.rotate or (math.ceil(2 * MALL_BYTES / (wbytes + M * K * esz)) + 1)
    log(f"device {torch.cuda.get_device_name(dev)}; workload {args.workload} M={M} K={K} N={N} "
        f"{act}; verify T={T} B={B}; rotating {R} copies ({R * wbytes / 1e6:.0f} MB)")

    xt = {"bf16": lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16),
          "fp16": lambda a: torch.from_numpy(a.view(np.int16)).view(torch.float16),
          "fp32": lambda a: torch.from_numpy(a)}[act]
    x0 = xt(c["x"][:M].copy()).to(dev)
    wq0 = torch.from_numpy(c["wq"]).to(dev)
    s0 = torch.from_numpy(c["scales"].view(np.int16)).view(torch.float16).to(dev)
    b0 = torch.from_numpy(c["biases"].view(np.int16)).view(torch.float16).to(dev)
    copies = [(x0, wq0, s0, b0)] + [(x0.clone(), wq0.clone(), s0.clone(), b0.clone())
                                    for _ in range(R - 1)]
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if T:
        rng = np.random.default_rng((c["seed"], 5))
        draft = torch.from_numpy(rng.integers(0, N, size=(B, max(T - 1, 1))).astype(np.int32)
                                 [:, :T - 1].copy()).to(dev)
        am = torch.empty(B * T, dtype=torch.int32, device=dev)
        al = torch.empty(B, dtype=torch.int32, device=dev)
        vws = torch.empty(max(vqv.vqv_verify_workspace_bytes(B, T, N), 8), dtype=torch.uint8,
                          device=dev)
    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        xc, wc, sc, bc = copies[i % R]
        if evs:
            evs[0].record(stream)
        vqv.vqv_qgemm(xc, wc, sc, bc, y=y, stream=stream)
        if evs:
            evs[1].record(stream)
        if T:
            vqv.vqv_verify(y, draft if T > 1 else None, B, T, argmax=am, accept_len=al,
                           workspace=vws, stream=stream)
            if evs:
                evs[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Whole-step throughput: K steps between two events, nothing else queued.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # Per-launch durations: events around each launch, on the launch stream.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    q_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    v_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evs] if T else [0.0]
    q_mean = statistics.fmean(q_us)

    qb = qgemm_bytes(M, K, N, esz)
    achieved = qb / (q_mean * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": M / (ms_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": act,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: W4 group-64 QMM M={M} K={K} N={N} {act} "
                               + (f"+ greedy verify B={B} T={T}" if T else "(no verify)"),
                   "M": M, "K": K, "N": N, "group": 64, "act": act, "verify_B": B,
                   "verify_T": T, "weight_copies": R},
        "qgemm_us_mean": q_mean,
        "qgemm_us_median": statistics.median(q_us),
        "verify_us_mean": statistics.fmean(v_us),
        "step_hbm_gbs": (qb + (4 * M * N if T else 0)) / (ms_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_record(args.workload, M),
                     "kernel": "qgemm_w4", "bytes_per_launch": qb},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(c, M, T, B, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
