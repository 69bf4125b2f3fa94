#!/usr/bin/env python3
"""Throughput of the W4 verify projection + greedy verify on one MI355X.

One step is the whole hot path over one verify block: the W4 QMM (group 64,
or 32 / 128 with --group) y[M,N] = x[M,K] . W^T, then the per-row argmax and accept walk over y. By
default a step is one vqv_qgemm_verify call (the argmax fused into the QMM
epilogue, a one-work-group kernel finishing the rows and the walk); with
--path separate it is vqv_qgemm followed by vqv_verify; with --path swiglu
(the gate/up workload) it is one vqv_qgemm_swiglu call, the projection of the
stacked gate/up weight with its silu-gated epilogue. The default workload
is the target projection M=8, K=5120, N=17408 with bf16 activations and a
verify block of T=8. Inputs are seeded synthetic tensors of that shape,
resident in HBM before timing. The weights rotate through enough copies that
every step streams them from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line. `value` is verified rows per second (M rows per step),
timed over the K steps captured as one HIP graph, so the host's launch cost
stays out of the measurement (the eagerly launched rate is reported beside
it). `roofline` reports the QMM kernel's algorithmic bytes per launch divided
by its mean launch time (HIP events around a graph of back-to-back QMM
launches, on the stream they run on) against the 8 TB/s HBM peak;
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
The step writes the logits y, as the plain projection does; on the fused
path the line also times the same call without them (y is optional there:
the argmax and accept lengths do not need it), `fused_no_logits_us_mean` and
`rows_per_s_no_logits`.

`--variant m8|m8q|v` pins the projection kernel family of the M <= 8 path
(through VQV_FORCE_VARIANT) so that a profiler trace holds one variant only.
On the target workload the line also carries the M=8 versus M=4 verified-row
throughput at K=5120, N=1024 (the shape of the pages' 1.811133x figure); on
the batched workload, the committed tokens per round with per-row accepts
against a round clamped to the shortest sequence, for drafts planted at
accept lengths drawn uniformly from 0..T-1.

Three further modes read rocprofv3 runs: `--counter-pass` launches the QMM
and a copy kernel of known size eagerly, `--write-traffic` turns a FETCH_SIZE
run and a WRITE_SIZE run of it (and optionally a run over the read request
counts by size, a check that needs no calibration) into per-launch HBM
bytes, and `--gap-report`
turns a kernel trace into a table of kernel durations and of the idle time
between consecutive dispatches (the GPU timeline's holes), per pair of
neighbouring kernels.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verified rows/s + achieved HBM GB/s, W4 M=8 QMM K=5120 N=17408"
MALL_BYTES = 256 << 20
COPY_PROBE_BYTES = 1 << 30
COPY_REF_BYTES = 512 << 20                     # the secondary bandwidth reference
QMM_LAUNCHES = 240

# workload -> (verify block T, sequences B) for the steps that include verify
VERIFY = {"tiny": (8, 1), "target": (8, 1), "vocab_verify": (8, 1), "batched_vocab": (16, 4)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def qgemm_bytes(M, K, N, esz, group=64):
    return K * N // 2 + 4 * N * (K // group) + M * K * esz + 4 * M * N


KERNEL_SOURCES = ("qgemm.hip", "qgemm_common.h", "qgemm_m16.hip", "qgemm_m8.hip",
                  "qgemm_v.hip")


def kernel_sha():
    """sha256 over the projection kernels' sources, in a fixed order."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "w4_gemm_vqv_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_key(workload, M, group, path="fused"):
    return (f"{workload}:M={M}" + ("" if group == 64 else f":group={group}")
            + (":swiglu" if path == "swiglu" else ""))


def traffic_record(workload, M, group=64, path="fused"):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs,
    valid only while the kernel source is unchanged."""
    fpath = os.path.join(ROOT, "profiles", "qgemm_traffic.json")
    if not os.path.exists(fpath):
        return None
    rec = json.load(open(fpath))
    entry = rec.get("workloads", {}).get(traffic_key(workload, M, group, path))
    if not entry or rec.get("kernel_sources_sha256") != kernel_sha():
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
        qgemm_ref(x, c["act"], c["wq"][:ncols], c["scales"][:ncols], c["biases"][:ncols],
                  c["group"])
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
    # One single-threaded pass over a smaller sample, for reference.
    t_1 = None
    try:
        from threadpoolctl import threadpool_limits
        n1 = max(64, ncols // 8)
        with threadpool_limits(limits=1, user_api="blas"):
            t_1 = run(n1) * N / n1
    except Exception:
        pass
    return {"value": M / (t_q + t_v), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"qgemm over {ncols} of {N} columns (median of 3, scaled to N) + "
                      f"verify over all {B * T} x {N} logits; host cpus {os.cpu_count()}",
            "seconds_per_step": t_q + t_v,
            "host_cpu_count": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0)),
            "blas_threads": threads,
            "single_thread_qgemm_rows_s": (M / t_1) if t_1 else None}


def _counter_rows(run_dir):
    """(kernel name, counter, value) rows of one rocprofv3 --pmc run, from its
    CSV output or its SQLite database."""
    import csv
    import glob
    import sqlite3
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    if rows:
        return rows
    for path in glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True):
        db = sqlite3.connect(path)
        rows += db.execute("select kernel_name, counter_name, value from counters_collection"
                           ).fetchall()
    if not rows:
        raise SystemExit(f"no counter records under {run_dir}")
    return rows


def _short_kernel(name):
    """A trace's kernel name without its namespace and argument list."""
    name = re.sub(r"^void ", "", name).replace("vqv::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def gap_report(run_dir):
    """Per pair of neighbouring dispatches (kernel A, then kernel B) in a
    rocprofv3 kernel trace (CSV output or SQLite database): how often it
    occurs, B's median duration and the median and 90th-percentile idle time
    from A's end to B's start (us)."""
    import csv
    import glob
    import sqlite3
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += [(r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                 for r in csv.DictReader(open(path))]
    if not rows:
        for path in glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True):
            db = sqlite3.connect(path)
            rows += db.execute("select name, start, end from kernels").fetchall()
    if not rows:
        raise SystemExit(f"no kernel records under {run_dir}")
    rows.sort(key=lambda r: r[1])
    pairs = {}
    for (a, _, a_end), (b, b_start, b_end) in zip(rows, rows[1:]):
        key = (_short_kernel(a), _short_kernel(b))
        d = pairs.setdefault(key, ([], []))
        d[0].append((b_end - b_start) / 1e3)
        d[1].append((b_start - a_end) / 1e3)
    out = []
    for (a, b), (dur, gap) in sorted(pairs.items(), key=lambda kv: -len(kv[1][0])):
        gap.sort()
        out.append({"after": a, "kernel": b, "count": len(dur),
                    "kernel_us_median": statistics.median(dur),
                    "gap_us_median": statistics.median(gap),
                    "gap_us_p90": gap[min(len(gap) - 1, int(0.9 * len(gap)))]})
    print(json.dumps(out, indent=1))


def _fused_kernel(kname):
    """The M <= 8 projection kernels' instances with the verify epilogue (the
    eighth template argument of qgemm_w4_m8, the fifth of qgemm_w4_m8q)."""
    for name, pos in (("qgemm_w4_m8<", 7), ("qgemm_w4_m8q<", 4)):
        if name in kname:
            args = kname.split(name, 1)[1].split(">", 1)[0].split(",")
            return len(args) > pos and args[pos].strip() == "true"
    return False


def _request_bytes(run_dir):
    """Read bytes per dispatch of a rocprofv3 --pmc pass over TCC_EA0_RDREQ_32B,
    _64B and _128B (CSV output): 32, 64 and 128 bytes per request of each size,
    summed over the instances. Returns (QMM dispatches, copy dispatches)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            size = {"TCC_EA0_RDREQ_32B": 32, "TCC_EA0_RDREQ_64B": 64,
                    "TCC_EA0_RDREQ_128B": 128}.get(r["Counter_Name"])
            if size is None:
                continue
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + size * float(r["Counter_Value"])
    q = [b for (_, k), b in sorted(per.items()) if "qgemm_w4" in k and not _fused_kernel(k)]
    cp = [b for (_, k), b in sorted(per.items()) if "neg" in k.lower()]
    if not q or not cp:
        raise SystemExit(f"no QMM or copy dispatches with request counts under {run_dir}")
    return q, cp


def write_traffic(fetch_dir, write_dir, workload, M, group=64, path="fused", req_dir=None):
    """Per-launch HBM bytes of the QMM from a FETCH_SIZE pass and a WRITE_SIZE
    pass of `bench.py --counter-pass`, each scaled by what the same counter
    reads for the copy kernel (COPY_PROBE_BYTES read and written per launch).
    With a third pass over the read request counts by size, the read bytes
    are also summed request by request, a check of the copy-kernel scaling
    that needs no calibration."""
    out = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        q, cp = [], []
        for kname, cname, v in _counter_rows(run_dir):
            if cname != counter:
                continue
            if "qgemm_w4" in kname and not _fused_kernel(kname):
                q.append(v)
            elif "neg" in kname.lower():
                cp.append(v)
        if not q or not cp:
            raise SystemExit(f"{counter}: no QMM or copy dispatches under {run_dir}")
        half = len(q) // 2  # the second sweep over the weight copies
        q_kib = statistics.fmean(q[half:])
        per_byte = statistics.fmean(cp) * 1024 / COPY_PROBE_BYTES
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        out[f"{key}_bytes"] = q_kib * 1024 / per_byte
        out[f"{key}_counter_kib"] = q_kib
        out[f"{key}_copy_calibration"] = per_byte
        out[f"{key}_dispatches"] = len(q) - half
    if req_dir:
        q, cp = _request_bytes(req_dir)
        out["read_bytes_by_request_size"] = statistics.fmean(q[len(q) // 2:])
        out["copy_read_bytes_by_request_size"] = statistics.fmean(cp)
    out_path = os.path.join(ROOT, "profiles", "qgemm_traffic.json")
    rec = json.load(open(out_path)) if os.path.exists(out_path) else {}
    sha = kernel_sha()
    if rec.get("kernel_sources_sha256") != sha:
        rec = {"kernel_sources_sha256": sha, "workloads": {}}
    key = traffic_key(workload, M, group, path)
    rec["workloads"][key] = out
    json.dump(rec, open(out_path, "w"), indent=1, sort_keys=True)
    print(json.dumps({key: out}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="target",
                    choices=["tiny", "target", "draft_w4a32", "vocab_verify", "batched_vocab",
                             "gate_up"])
    ap.add_argument("--m", type=int, default=None, help="rows (default: the workload's M)")
    ap.add_argument("--n", type=int, default=None,
                    help="output columns (default: the workload's N), e.g. one GPU's column "
                         "share of a sharded projection")
    ap.add_argument("--group", type=int, choices=[32, 64, 128], default=64,
                    help="k per scale and bias (the workloads are quoted at 64)")
    ap.add_argument("--rotate", type=int, default=None, help="weight copies cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["fused", "separate", "swiglu"], default="fused",
                    help="one step: the projection with the verify fused into its epilogue, "
                         "the two calls back to back, or (gate/up) the projection with its "
                         "SwiGLU epilogue")
    ap.add_argument("--variant", choices=["auto", "m8", "m8q", "v"], default="auto",
                    help="pin the M <= 8 projection kernel (sets VQV_FORCE_VARIANT): m8q is "
                         "the whole-line MFMA kernel, m8 the half-line one, v the vector-ALU "
                         "kernel (one or two rows)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="eager QMM launches + a copy kernel, for one rocprofv3 --pmc pass")
    ap.add_argument("--write-traffic", nargs="+", metavar="DIR",
                    help="summarize --counter-pass runs into profiles/qgemm_traffic.json: "
                         "FETCH_SIZE dir, WRITE_SIZE dir [, TCC_EA0_RDREQ_32B/64B/128B dir]")
    ap.add_argument("--gap-report", metavar="TRACE_DIR",
                    help="kernel durations and idle gaps between neighbouring dispatches "
                         "of a rocprofv3 --kernel-trace run")
    args = ap.parse_args()
    if args.gap_report:
        gap_report(args.gap_report)
        return
    if args.write_traffic:
        import gen
        if len(args.write_traffic) not in (2, 3):
            raise SystemExit("--write-traffic takes FETCH_DIR WRITE_DIR [REQUEST_DIR]")
        fdir, wdir, *rdir = args.write_traffic
        write_traffic(fdir, wdir, args.workload, args.m or gen.CONFIGS[args.workload]["M"],
                      args.group, args.path, rdir[0] if rdir else None)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py measures one GPU only: the library has no multi-GPU path "
                  f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    if args.variant != "auto":
        os.environ["VQV_FORCE_VARIANT"] = args.variant
    import numpy as np
    import torch

    import gen
    import w4_gemm_vqv_amd as vqv

    vqv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = gen.make_config(args.workload, group=args.group,
                        **({"N": args.n} if args.n else {}))
    M = args.m or c["M"]
    K, N, act = c["K"], c["N"], c["act"]
    esz = 4 if act == "fp32" else 2
    vqv_act = {"bf16": 0, "fp16": 1, "fp32": 2}[act]
    T, B = VERIFY.get(args.workload, (0, 0))
    if T:
        if B == 1:
            T = M
        elif B * T != M:
            raise SystemExit(f"{args.workload}: M must be {B * T}")

    group = args.group
    wbytes = K * N // 2 + 4 * N * (K // group)
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
        if B > 1:
            # Drafts planted around the library's own argmax at accept
            # lengths drawn from 0..T-1, so that the rounds' accept counts
            # vary per sequence (the batched workload's recipe).
            a0 = vqv.vqv_verify(vqv.vqv_qgemm(x0, wq0, s0, b0, group=args.group),
                                draft, B, T)[0].cpu().numpy()
            planted = rng.integers(0, T, size=B)
            draft = torch.from_numpy(gen.make_drafts(a0, B, T, N, seed=c["seed"],
                                                     accept=planted).astype(np.int32)).to(dev)
        am = torch.empty(B * T, dtype=torch.int32, device=dev)
        al = torch.empty(B, dtype=torch.int32, device=dev)
        vws = torch.empty(max(vqv.vqv_verify_workspace_bytes(B, T, N), 8), dtype=torch.uint8,
                          device=dev)
    stream = torch.cuda.current_stream()
    fused_ok = T > 0 and vqv.vqv_qgemm_verify_workspace_bytes(M, K, N, group, vqv_act) > 0
    if fused_ok:
        fws = torch.zeros(vqv.vqv_qgemm_verify_workspace_bytes(M, K, N, group, vqv_act),
                          dtype=torch.uint8, device=dev)
    use_fused = fused_ok and args.path == "fused"
    use_swiglu = args.path == "swiglu"
    if use_swiglu:
        if T or N % 2:
            raise SystemExit("--path swiglu takes a gate/up workload (even N, no verify)")
        hbuf = torch.empty((M, N // 2), dtype=torch.float32, device=dev)
        sws_n = vqv.vqv_qgemm_swiglu_workspace_bytes(M, K, N, group, vqv_act)
        sws = torch.empty(sws_n, dtype=torch.uint8, device=dev) if sws_n else None

    def qmm(i, st):
        xc, wc, sc, bc = copies[i % R]
        vqv.vqv_qgemm(xc, wc, sc, bc, y=y, group=group, stream=st)

    def ver(st):
        vqv.vqv_verify(y, draft if T > 1 else None, B, T, argmax=am, accept_len=al,
                       workspace=vws, stream=st)

    def fused(i, st):
        xc, wc, sc, bc = copies[i % R]
        vqv.vqv_qgemm_verify(xc, wc, sc, bc, draft if T > 1 else None, B, T, y=y, argmax=am,
                             accept_len=al, workspace=fws, group=group, stream=st)

    def swiglu(i, st):
        xc, wc, sc, bc = copies[i % R]
        vqv.vqv_qgemm_swiglu(xc, wc, sc, bc, h=hbuf, workspace=sws, group=group, stream=st)

    def step(i, st):
        if use_fused:
            fused(i, st)
            return
        if use_swiglu:
            swiglu(i, st)
            return
        qmm(i, st)
        if T:
            ver(st)

    if args.counter_pass:
        # Eager launches for rocprofv3 --pmc (one counter pass per run): the
        # QMM (with --path swiglu the gate/up projection with its SwiGLU
        # epilogue) over every weight copy twice, then a plain copy kernel of
        # known size whose counter reading calibrates bytes per counted unit.
        for i in range(2 * R):
            (swiglu if use_swiglu else qmm)(i, stream)
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"counter pass done: {2 * R} QMM launches, 3 copy launches of "
            f"{COPY_PROBE_BYTES} bytes each way")
        return

    def graph_of(fn, n):
        """HIP graph of n launches of fn(i, stream); launch overhead of the
        Python binding stays out of the timed region."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for i in range(n):
                fn(i, cs)
        return g

    def timed(g, reps=1):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()

    # Whole-step throughput: the K steps as one graph, replayed once untimed
    # (upload) and once timed, with nothing else queued.
    g_steps = graph_of(step, args.steps)
    for _ in range(3):                  # upload, then clocks and caches in steady state
        g_steps.replay()
    ms_step = timed(g_steps) / args.steps

    # The same K steps launched one by one from Python, for reference.
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1) / args.steps

    # Per-launch durations: back-to-back launches of one kernel in a graph,
    # HIP events around the replays on the stream the kernels run on.
    nq = R * max(1, math.ceil(QMM_LAUNCHES / R))
    g_q = graph_of(qmm, nq)
    g_q.replay()
    q_runs = [timed(g_q) * 1e3 / nq for _ in range(5)]
    q_mean = statistics.fmean(q_runs)
    v_runs = [0.0]
    if T:
        g_v = graph_of(lambda i, st: ver(st), QMM_LAUNCHES)
        g_v.replay()
        v_runs = [timed(g_v) * 1e3 / QMM_LAUNCHES for _ in range(5)]
    s_runs = None
    if use_swiglu:
        g_s = graph_of(swiglu, nq)
        g_s.replay()
        s_runs = [timed(g_s) * 1e3 / nq for _ in range(5)]
    f_runs = None
    fn_runs = None
    if use_fused:
        g_f = graph_of(fused, nq)
        g_f.replay()
        f_runs = [timed(g_f) * 1e3 / nq for _ in range(5)]

        # The same fused call without the logits: y is not written, and the
        # argmax and accept lengths are the same (the fused verify needs no
        # logits; the step above writes them, as the plain projection does).
        def fused_no_logits(i, st):
            xc, wc, sc, bc = copies[i % R]
            vqv.vqv_qgemm_verify(xc, wc, sc, bc, draft if T > 1 else None, B, T, y=None,
                                 want_y=False, argmax=am, accept_len=al, workspace=fws,
                                 group=group, stream=st)

        g_fn = graph_of(fused_no_logits, nq)
        g_fn.replay()
        fn_runs = [timed(g_fn) * 1e3 / nq for _ in range(5)]

    # Secondary bandwidth reference: a device copy of 512 MiB each way,
    # timed the same way (graph of back-to-back copies).
    csrc = torch.empty(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    g_c = graph_of(lambda i, st: cdst.copy_(csrc), 4)
    g_c.replay()
    copy_gbs = 2 * COPY_REF_BYTES * 4 / (min(timed(g_c) for _ in range(3)) * 1e-3) / 1e9
    # Read-only context: torch's own sum over 1 GiB (it writes 4 bytes). It
    # reads at about 3.9-4.0 TB/s here, below what the copy and the projection
    # kernels stream, so it is reported as context and no fraction is taken of
    # it. Launched eagerly (the reduction may clear memory with memsets, which
    # stay out of graphs); four back-to-back sums between events.
    rsrc = torch.empty(2 * COPY_REF_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    torch.sum(rsrc)
    r_ms = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(4):
            torch.sum(rsrc)
        e1.record(stream)
        torch.cuda.synchronize()
        r_ms.append(e0.elapsed_time(e1))
    read_gbs = 4 * 2 * COPY_REF_BYTES / (min(r_ms) * 1e-3) / 1e9
    del csrc, cdst, g_c, rsrc

    # Rows/s against M with the same weights (the first M rows of x): the
    # plain projection's per-launch time at M = 1 and 4 as well.
    by_m, n1024 = {}, None
    if args.workload == "target" and M == c["M"]:
        for m_sub in (1, 4):
            xs_sub = [cp[0][:m_sub].contiguous() for cp in copies]
            ys_sub = torch.empty((m_sub, N), dtype=torch.float32, device=dev)

            def qm(i, st, xs_sub=xs_sub, ys_sub=ys_sub):
                _, wc, sc, bc = copies[i % R]
                vqv.vqv_qgemm(xs_sub[i % R], wc, sc, bc, y=ys_sub, group=group, stream=st)
            g_m = graph_of(qm, nq)
            g_m.replay()
            t_m = statistics.fmean(timed(g_m) * 1e3 / nq for _ in range(3))
            by_m[m_sub] = {"us_per_launch": t_m, "rows_per_s": m_sub / (t_m * 1e-6)}
        by_m[M] = {"us_per_launch": q_mean, "rows_per_s": M / (q_mean * 1e-6)}
        # The pages' figure is measured at K=5120, N=1024: the same K with a
        # narrow output, rotated past the Infinity Cache.
        rng_n = np.random.default_rng((c["seed"], 1024))
        wn, sn, bn = gen.make_weights(rng_n, 1024, K, group)
        Rn = math.ceil(2 * MALL_BYTES / (1024 * K // 2 + 4 * 1024 * (K // group))) + 1
        narrow = [(torch.from_numpy(wn).to(dev),
                   torch.from_numpy(sn.view(np.int16)).view(torch.float16).to(dev),
                   torch.from_numpy(bn.view(np.int16)).view(torch.float16).to(dev))
                  for _ in range(Rn)]
        n1024 = {}
        for m_sub in (4, 8):
            xs_n = x0[:m_sub].contiguous()
            ys_n = torch.empty((m_sub, 1024), dtype=torch.float32, device=dev)

            def qn(i, st, xs_n=xs_n, ys_n=ys_n):
                wc, sc, bc = narrow[i % Rn]
                vqv.vqv_qgemm(xs_n, wc, sc, bc, y=ys_n, group=group, stream=st)
            ln = Rn * max(1, math.ceil(QMM_LAUNCHES / Rn))
            g_n = graph_of(qn, ln)
            g_n.replay()
            t_n = statistics.fmean(timed(g_n) * 1e3 / ln for _ in range(3))
            n1024[m_sub] = {"us_per_launch": t_n, "rows_per_s": m_sub / (t_n * 1e-6)}
        n1024["m8_over_m4_rows"] = n1024[8]["rows_per_s"] / n1024[4]["rows_per_s"]
        n1024["pages_m8_over_m4_rows"] = 1.811133
        del narrow

    clamp = None
    if T and B > 1:
        ver(stream)
        torch.cuda.synchronize()
        acc = al.cpu().numpy().astype(int)
        # Committed tokens per round: every sequence keeps its own accept count
        # plus its bonus token, against a round clamped to the shortest one.
        clamp = {"accept_len": acc.tolist(), "min_accept_len": int(acc.min()),
                 "tokens_per_round_per_row": int((acc + 1).sum()),
                 "tokens_per_round_clamped": int(B * (acc.min() + 1))}

    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "cus": props.multi_processor_count,
              "arch": getattr(props, "gcnArchName", None),
              "memory_gib": round(props.total_memory / 2 ** 30, 1),
              "hip": torch.version.hip, "torch": torch.__version__}

    qb = qgemm_bytes(M, K, N, esz, group)
    # The dominant kernel is the projection. Its launches are timed in a graph
    # of their own (the fused step's instance adds only the per-group argmax
    # epilogue, 8 bytes per row and work-group, and is timed with the finish
    # kernel in fused_us_mean).
    k_us = q_mean
    kname = vqv.vqv_qgemm_kernel(M, K, N, group, vqv_act)
    if use_swiglu:
        # The step's kernel is the projection with the SwiGLU epilogue: it
        # writes h [M, N/2] instead of y [M, N].
        qb = qb - 4 * M * N + 4 * M * (N // 2)
        k_us = statistics.fmean(s_runs)
        if kname == "qgemm_w4_m16":
            kname = "qgemm_w4_m16 (SwiGLU)"
    achieved = qb / (k_us * 1e-6) / 1e9
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
        "config": {"workload": f"{args.workload}: W4 group-{group} QMM M={M} K={K} N={N} {act} "
                               + (f"+ greedy verify B={B} T={T}" if T else "(no verify)")
                               + (" (verify fused into the QMM epilogue)" if use_fused
                                  else "")
                               + (" with the SwiGLU epilogue, h[M, N/2]" if use_swiglu else ""),
                   "M": M, "K": K, "N": N, "group": group, "act": act, "verify_B": B,
                   "verify_T": T, "weight_copies": R},
        "eager_ms_per_step": ms_eager,
        "qgemm_us_mean": q_mean,
        "qgemm_us_runs": q_runs,
        "verify_us_mean": statistics.fmean(v_runs),
        "fused_us_mean": statistics.fmean(f_runs) if f_runs else None,
        "fused_no_logits_us_mean": statistics.fmean(fn_runs) if fn_runs else None,
        "rows_per_s_no_logits": M / (statistics.fmean(fn_runs) * 1e-6) if fn_runs else None,
        "swiglu_us_mean": statistics.fmean(s_runs) if s_runs else None,
        "step_path": "fused" if use_fused else ("swiglu" if use_swiglu else "separate"),
        "step_hbm_gbs": (qb + (4 * M * N if T and not use_fused else 0)) / (ms_step * 1e-3) / 1e9,
        # The step's own projection instance carries the argmax epilogue and is
        # followed by the finishing kernel: the fused call's mean launch time
        # bounds it from above (rocprofv3 separates the two kernels).
        "fused_call_frac": (qb / (statistics.fmean(f_runs) * 1e-6) / 1e9 / HBM_PEAK_GBS
                            if f_runs else None),
        "device": device,
        "copy_probe_gbs": copy_gbs,
        "torch_sum_read_gbs": read_gbs,
        "qgemm_by_M": by_m or None,
        "k5120_n1024_by_M": n1024,
        "batched_accepts": clamp,
        "variant": args.variant,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "frac_of_copy_probe": achieved / copy_gbs,
                     "traffic": None if args.n else
                                traffic_record(args.workload, M, group, args.path),
                     "kernel": kname, "bytes_per_launch": qb, "us_per_launch": k_us},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(c, M, T, B, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
