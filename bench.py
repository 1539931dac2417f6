#!/usr/bin/env python3
"""Attention backward benchmark on one MI355X.

One step = one full backward pass (preprocess -> dK/dV -> dQ, every kernel of
the path) over one batch of seeded synthetic inputs already resident in HBM;
O and LSE come from one untimed forward.  Prints ONE JSON line on stdout:

  metric/value/unit    backward TFLOP/s, counted as 10*b*h*Sq*Sk*d (halved
                       when causal), over the MEDIAN of K hipEvent-bracketed
                       attn_bwd calls on the launch stream (the mean and the
                       wall clock of the K calls, bracketed by
                       torch.cuda.synchronize(), are reported beside it);
  roofline             the dominant kernel (dK/dV) against the MI355X dense
                       fp16/bf16 matrix-core peak, its duration the median of
                       HIP events around that kernel's launch on the launch
                       stream; HBM traffic from the committed rocprofv3
                       FETCH_SIZE/WRITE_SIZE measurement when it still matches
                       the kernel source (else null);
  forward              the forward kernel that supplies O and LSE, timed the
                       same way (not part of the metric);
  cpu_baseline         the fp64 CPU oracle's backward on a bounded sample of
                       the same workload (whole heads), scaled to TFLOP/s.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 40] [--workload NAME]
       python bench.py --calibrate     (matrix-core / LDS / atomic rates of the box)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

MFMA_PEAK_TFLOPS = {"fp16": 2516.6, "bf16": 2516.6}  # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
# What bench_calibrate.hip's products-only loop sustains on an MI355X (8 waves
# per CU); profiles/calibration_mi355x.md.  Context for the roofline
# fraction, not its denominator.
MFMA_MEASURED_TFLOPS = {"fp16": 2469.0, "bf16": 2469.0}
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["flashattention_backward_pass_attn_amd/csrc/attn_bwd_split.h",
                  "flashattention_backward_pass_attn_amd/csrc/attn_bwd_dq.h",
                  "flashattention_backward_pass_attn_amd/csrc/attn_bwd.h",
                  "flashattention_backward_pass_attn_amd/csrc/attn_fwd.h",
                  "flashattention_backward_pass_attn_amd/csrc/attn_device.h"]
TRAFFIC_FILE = "profiles/{kernel}_traffic_{workload}.json"
# Matrix-core work of each gradient kernel, in units of 2*b*h*Sq*Sk*d (halved
# when causal): dK/dV does S, dP, dV, dK; dQ recomputes S and dP and does dQ.
# The metric counts the method's 5 contractions (10*b*h*Sq*Sk*d) for the whole
# backward; the 2 recomputed ones are not counted.
KERNEL_UNITS = {"attn_bwd_dkdv_kernel": 4, "attn_bwd_dq_kernel": 3}
# launch name of each gradient kernel's symbol, per head-dim tile
DQ_SYMBOL = {False: "attn_bwd_dq_recompute_kernel", True: "attn_bwd_dq_wide_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def workload_flops(w: workloads.Workload, inp) -> float:
    if w.varlen:
        return workloads.attention_flops(w.batch, w.heads_q, 0, 0, w.head_dim, w.causal,
                                         lengths=[int(x) for x in inp["lengths_q"]])
    return workloads.attention_flops(w.batch, w.heads_q, w.seqlen, w.seqlen, w.head_dim, w.causal)


def load_traffic(workload: str, kernel: str):
    path = os.path.join(ROOT, TRAFFIC_FILE.format(workload=workload, kernel=kernel))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_sha():
        log(f"traffic record {path} predates the current kernel source: reporting null")
        return None
    return rec


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w: workloads.Workload, inp, budget_s: float):
    """Time the oracle backward (given the oracle's own LSE) on whole heads until ~budget_s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    scale = 1.0 / math.sqrt(w.head_dim)
    G = w.heads_q // w.heads_kv
    done_flops, spent, heads = 0.0, 0.0, 0
    # sample: query heads of sequence 0 in order (varlen: the sequences in order)
    order = []
    nseq = len(inp["lengths_q"]) if w.varlen else w.batch
    for z in range(nseq):
        for h in range(w.heads_q):
            order.append((z, h))
    for z, h in order:
        if w.varlen:
            a, e = int(inp["cu_seqlens_q"][z]), int(inp["cu_seqlens_q"][z + 1])
            q, k, v, do = (inp[n][a:e] for n in ("q", "k", "v", "do"))
            L = e - a
            fl = workloads.attention_flops(1, 1, 0, 0, w.head_dim, w.causal, lengths=[L])
            qh, kh, vh, doh = q[:, h], k[:, h // G], v[:, h // G], do[:, h]
        else:
            qh, kh, vh, doh = (inp[n][z, :, hh] for n, hh in (("q", h), ("k", h // G), ("v", h // G), ("do", h)))
            fl = workloads.attention_flops(1, 1, w.seqlen, w.seqlen, w.head_dim, w.causal)
        qh, kh, vh, doh = (np.asarray(x, dtype=np.float64) for x in (qh, kh, vh, doh))
        _, lse = oracle.head_forward(qh, kh, vh, scale, w.causal)  # untimed: supplies LSE
        t0 = time.perf_counter()
        oracle.head_backward(qh, kh, vh, doh, scale, w.causal, lse=lse)
        spent += time.perf_counter() - t0
        done_flops += fl
        heads += 1
        if spent >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": done_flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "host_cpu": host_cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{heads} (sequence, query head) pairs of {w.name}, fp64 NumPy backward given the oracle's "
                  f"LSE, {spent:.1f} s; flops counted as for the GPU",
        "seconds": round(spent, 3),
    }


COPY_BYTES = 1 << 30  # the --copy-calibration copy: 1 GiB read and 1 GiB written per launch
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_rows(path: str, counter: str):
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                # "void ns::name<targs>(args)" -> "name"; both dQ kernels count as the dQ kernel
                name = r["Kernel_Name"].split("(")[0].split("<")[0].split()[-1].split("::")[-1]
                if name in DQ_SYMBOL.values():
                    name = "attn_bwd_dq_kernel"
                rows.setdefault(name, []).append(float(r["Counter_Value"]))
    return rows


def write_traffic(fetch_csv: str, write_csv: str, workload: str, command: str) -> int:
    """Turn two rocprofv3 --pmc runs of `bench.py --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, both
    in KiB per dispatch) into per-launch HBM bytes for each gradient kernel.  Each counter is scaled by
    what it reads for a plain 1 GiB device copy in the same run."""
    fetch, write = _counter_rows(fetch_csv, "FETCH_SIZE"), _counter_rows(write_csv, "WRITE_SIZE")
    if COPY_KERNEL not in fetch or COPY_KERNEL not in write:
        log(f"no {COPY_KERNEL} rows: run the profiled bench with --copy-calibration")
        return 1
    f_factor = COPY_BYTES / (sum(fetch[COPY_KERNEL]) / len(fetch[COPY_KERNEL]) * 1024)
    w_factor = COPY_BYTES / (sum(write[COPY_KERNEL]) / len(write[COPY_KERNEL]) * 1024)
    for kernel in [*KERNEL_UNITS, "attn_fwd_kernel"]:
        if kernel not in fetch or kernel not in write:
            log(f"{kernel}: missing from the counter files")
            return 1
        fk = sum(fetch[kernel]) / len(fetch[kernel])
        wk = sum(write[kernel]) / len(write[kernel])
        rec = {
            "workload": workload, "kernel": kernel, "source_sha256": kernel_source_sha(),
            "command": command,
            "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
            "dispatches": [len(fetch[kernel]), len(write[kernel])],
            "copy_fetch_factor": round(f_factor, 4), "copy_write_factor": round(w_factor, 4),
            "hbm_read_bytes_per_launch": round(fk * 1024 * f_factor),
            "hbm_write_bytes_per_launch": round(wk * 1024 * w_factor),
        }
        rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
        short = kernel.replace("attn_bwd_", "").replace("attn_", "").replace("_kernel", "")
        out = os.path.join(ROOT, TRAFFIC_FILE.format(workload=workload, kernel=short))
        os.makedirs(os.path.dirname(out), exist_ok=True)
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        log(f"{out}: {rec['hbm_bytes_per_launch'] / 1e9:.3f} GB per launch "
            f"(factors fetch {f_factor:.3f}, write {w_factor:.3f})")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=workloads.DEFAULT_BENCH_WORKLOAD, choices=sorted(workloads.ALL_WORKLOADS))
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the per-launch HBM traffic records from two rocprofv3 --pmc counter_collection "
                         "files (FETCH_SIZE, WRITE_SIZE) of `bench.py --copy-calibration`, then exit")
    ap.add_argument("--traffic-command", default="",
                    help="with --traffic-from: the profiled command, stored in the record")
    ap.add_argument("--calibrate", action="store_true",
                    help="build and run bench_calibrate.hip (matrix-core, LDS, vector-overlap and atomic rates)")
    args = ap.parse_args(argv)

    if args.calibrate:
        return calibrate()
    if args.traffic_from:
        return write_traffic(args.traffic_from[0], args.traffic_from[1], args.workload, args.traffic_command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the backward is independent "
              "per (batch, head), so more GPUs would each run this same kernel on their share; no "
              "multi-GPU figure is produced.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import flashattention_backward_pass_attn_amd as fa

    w = workloads.ALL_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workloads.make_workload_inputs(w.name)
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def up(n):
        return torch.from_numpy(np.ascontiguousarray(inp[n + "_bits"]).view(np.int16)).view(tdt).to(dev)

    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    kw = {}
    if w.varlen:
        kw = dict(cu_seqlens_q=torch.from_numpy(inp["cu_seqlens_q"]).to(dev),
                  cu_seqlens_k=torch.from_numpy(inp["cu_seqlens_k"]).to(dev),
                  max_seqlen_q=int(inp["lengths_q"].max()), max_seqlen_k=int(inp["lengths_k"].max()))
    scale = 1.0 / math.sqrt(w.head_dim)
    o, lse = fa.attn_fwd(q, k, v, causal=w.causal, softmax_scale=scale, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    p = fa.make_params(q, k, w.causal, scale, args.deterministic, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"),
                       kw.get("max_seqlen_q"), kw.get("max_seqlen_k"))
    ws_bytes = fa.bwd_workspace_size(p)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    common = dict(causal=w.causal, softmax_scale=scale, deterministic=args.deterministic, dq=dq, dk=dk, dv=dv,
                  workspace=ws, **kw)
    flops = workload_flops(w, inp)
    torch.cuda.synchronize()

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    for _ in range(args.warmup):
        fa.attn_bwd(q, k, v, o, lse, do, **common)
    torch.cuda.synchronize()

    # Timed region: K full backward calls, each bracketed by HIP events on the
    # launch stream (the binding launches on torch's current stream).
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        fa.attn_bwd(q, k, v, o, lse, do, **common)
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = [a_.elapsed_time(b_) for a_, b_ in ev]
    ms_per_step = med(step_ms)
    ms_mean = sum(step_ms) / K
    ms_wall = (t1 - t0) * 1e3 / K
    log(f"{w.name}: step median {ms_per_step:.4f} ms, mean {ms_mean:.4f} ms, wall {ms_wall:.4f} ms per call")

    # Per-kernel durations: the same backward launched phase by phase (the dQ
    # kernel, which also runs the preprocess for its rows, then dK/dV), with
    # events between the launches (medians over as many steps).
    P = max(1, min(K, 50))
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(P)]
    for i in range(P):
        e = pev[i]
        e[0].record()
        fa.attn_bwd(q, k, v, o, lse, do, phases=fa.PHASE_DQ, **common)
        e[1].record()
        fa.attn_bwd(q, k, v, o, lse, do, phases=fa.PHASE_DKDV, **common)
        e[2].record()
    torch.cuda.synchronize()
    dq_ms = med([e[0].elapsed_time(e[1]) for e in pev])
    dkdv_ms = med([e[1].elapsed_time(e[2]) for e in pev])
    log(f"{w.name}: kernels dq (with the preprocess) {dq_ms:.4f} dkdv {dkdv_ms:.4f} ms")

    # The forward that supplies O and LSE (not part of the metric).
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for _ in range(5):
        fa.attn_fwd(q, k, v, causal=w.causal, softmax_scale=scale, out=o, lse=lse, **kw)
    for a_, b_ in fev:
        a_.record()
        fa.attn_fwd(q, k, v, causal=w.causal, softmax_scale=scale, out=o, lse=lse, **kw)
        b_.record()
    torch.cuda.synchronize()
    fwd_ms = med([a_.elapsed_time(b_) for a_, b_ in fev])

    if args.copy_calibration:
        n = 1 << 28  # 256 Mi floats = 1 GiB read + 1 GiB written
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} bytes read and written per copy kernel, 2 launches")

    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    kernels = {"attn_bwd_dkdv_kernel": dkdv_ms, "attn_bwd_dq_kernel": dq_ms}
    per_kernel = {}
    for name, ms in kernels.items():
        kfl = flops / 5.0 * KERNEL_UNITS[name]
        per_kernel[name] = {"ms": round(ms, 4), "tflops": round(kfl / (ms * 1e-3) / 1e12, 2),
                            "frac": round(kfl / (ms * 1e-3) / 1e12 / peak, 4), "flop": kfl, "bound": "mfma",
                            "contractions": KERNEL_UNITS[name]}
    per_kernel["attn_bwd_dq_kernel"]["symbol"] = DQ_SYMBOL[w.head_dim > 128]
    per_kernel["attn_bwd_dq_kernel"]["includes"] = "the preprocess of its rows (Delta, LSE*log2(e))"
    dom = max(kernels, key=kernels.get)
    traffic = load_traffic(w.name, dom.replace("attn_bwd_", "").replace("_kernel", ""))
    roofline = {
        "bound": "mfma",
        "achieved": per_kernel[dom]["tflops"],
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": per_kernel[dom]["frac"],
        "traffic": None if traffic is None else traffic["hbm_bytes_per_launch"],
        "kernel": dom,
        "kernel_ms": per_kernel[dom]["ms"],
        "kernels": per_kernel,
        "measured_peak": MFMA_MEASURED_TFLOPS[w.dtype],
        "frac_of_measured_peak": round(per_kernel[dom]["tflops"] / MFMA_MEASURED_TFLOPS[w.dtype], 4),
    }
    fwd_flops = flops * 0.4  # S = Q K^T and O = P V: 4*b*h*Sq*Sk*d, halved when causal
    forward = {"ms": round(fwd_ms, 4), "tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
               "frac": round(fwd_flops / (fwd_ms * 1e-3) / 1e12 / peak, 4), "flop": fwd_flops,
               "kernel": "attn_fwd_kernel", "bound": "mfma"}
    fwd_traffic = load_traffic(w.name, "fwd")
    forward["traffic"] = None if fwd_traffic is None else fwd_traffic["hbm_bytes_per_launch"]
    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("cpu baseline: timing the oracle backward on a bounded sample ...")
        cpu = cpu_baseline(w, inp, args.cpu_baseline_seconds)
    cfg = {"workload": w.name, "dtype": w.dtype, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
           "seqlen": (int(inp["lengths_q"].max()) if w.varlen else w.seqlen), "head_dim": w.head_dim,
           "causal": w.causal, "varlen": w.varlen, "deterministic": args.deterministic,
           "flop_per_step": flops, "workspace_bytes": ws_bytes, "parallelism": "single GPU"}
    if w.varlen:
        cfg["lengths"] = [int(x) for x in inp["lengths_q"]]
    rec = {
        "metric": "attention backward TFLOP/s (fp16/bf16, causal+non-causal) and % MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "ms_per_step_wall": round(ms_wall, 4),
        "timing": "median of K hipEvent-bracketed attn_bwd calls on the launch stream",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, see workloads/)",
        "config": cfg,
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "roofline": roofline,
        "forward": forward,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def calibrate() -> int:
    """Build bench_calibrate.hip with hipcc and run it (prints its table)."""
    import shutil
    import subprocess
    import tempfile
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    src = os.path.join(ROOT, "bench_calibrate.hip")
    out = os.path.join(tempfile.mkdtemp(prefix="attn_calibrate_"), "calibrate")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        return res.returncode
    return subprocess.run([out]).returncode


if __name__ == "__main__":
    sys.exit(main())
