#!/usr/bin/env python3
"""Attention backward benchmark on one MI355X.

One step = one full backward pass (preprocess -> main -> postprocess) over one
batch of seeded synthetic inputs already resident in HBM; O and LSE come from
one untimed forward.  Prints ONE JSON line on stdout:

  metric/value/unit    backward TFLOP/s, counted as 10*b*h*Sq*Sk*d (halved
                       when causal), over the wall clock of K steps bracketed
                       by torch.cuda.synchronize();
  roofline             the main kernel (the dominant one) against the MI355X
                       dense fp16/bf16 matrix-core peak, its duration taken
                       with HIP events on the launch stream inside the timed
                       region; HBM traffic from the committed rocprofv3
                       FETCH_SIZE/WRITE_SIZE measurement when it still matches
                       the kernel source (else null);
  cpu_baseline         the fp64 CPU oracle's backward on a bounded sample of
                       the same workload (a few heads), scaled to TFLOP/s.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 40] [--workload NAME]
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
# What flashattention_backward_pass_attn_amd/csrc/mfma_peak.hip sustains on an
# MI355X with nothing but 32x32x16 products in flight (clock about 1.93 GHz
# under that load); profiles/mfma_rate_and_valu_overlap_mi355x.md.  Context
# for the roofline fraction, not its denominator.
MFMA_MEASURED_TFLOPS = {"fp16": 1905.1, "bf16": 2026.2}
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["flashattention_backward_pass_attn_amd/csrc/attn_bwd_split.h",
                  "flashattention_backward_pass_attn_amd/csrc/attn_bwd_dq.h",
                  "flashattention_backward_pass_attn_amd/csrc/attn_device.h"]
TRAFFIC_FILE = "profiles/bwd_{kernel}_traffic_{workload}.json"
# Matrix-core work of each gradient kernel, in units of 2*b*h*Sq*Sk*d (halved
# when causal): dK/dV does S, dP, dV, dK; dQ (over the stored dS, the path the
# default workspace selects) does dQ only.  The metric counts the method's 5
# contractions (10*b*h*Sq*Sk*d) for the whole backward.
KERNEL_UNITS = {"attn_bwd_dkdv_kernel": 4, "attn_bwd_dq_kernel": 1}


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
                # "void ns::name<targs>(args)" -> "name"
                name = r["Kernel_Name"].split("(")[0].split("<")[0].split()[-1].split("::")[-1]
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
    for kernel in KERNEL_UNITS:
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
        short = kernel.replace("attn_bwd_", "").replace("_kernel", "")
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
    args = ap.parse_args(argv)

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
    ws = torch.empty(max(fa.bwd_workspace_size(p), 256), dtype=torch.uint8, device=dev)
    common = dict(causal=w.causal, softmax_scale=scale, deterministic=args.deterministic, dq=dq, dk=dk, dv=dv,
                  workspace=ws, **kw)
    flops = workload_flops(w, inp)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        fa.attn_bwd(q, k, v, o, lse, do, **common)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record()
        fa.attn_bwd(q, k, v, o, lse, do, phases=fa.PHASE_PREPROCESS, **common)
        e[1].record()
        fa.attn_bwd(q, k, v, o, lse, do, phases=fa.PHASE_DKDV, **common)
        e[2].record()
        fa.attn_bwd(q, k, v, o, lse, do, phases=fa.PHASE_DQ, **common)
        e[3].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    dkdv_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    dq_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    log(f"{w.name}: step {ms_per_step:.4f} ms (events: pre {pre_ms:.4f} dkdv {dkdv_ms:.4f} dq {dq_ms:.4f} ms)")

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
                            "frac": round(kfl / (ms * 1e-3) / 1e12 / peak, 4), "flop": kfl}
    # the dQ kernel streams the stored dS (2 bytes per visible (query, key)
    # pair = 2 * flops / (10 * d)) plus K and dQ once: HBM-bound
    elem = 2
    k_bytes = elem * w.head_dim * (int(inp["lengths_k"].sum()) * w.heads_kv if w.varlen
                                   else w.batch * w.seqlen * w.heads_kv)
    q_bytes = elem * w.head_dim * (int(inp["lengths_q"].sum()) * w.heads_q if w.varlen
                                   else w.batch * w.seqlen * w.heads_q)
    dq_bytes = elem * flops / (10.0 * w.head_dim) + k_bytes + q_bytes
    per_kernel["attn_bwd_dq_kernel"].update({
        "bound": "hbm", "bytes": dq_bytes,
        "gbs": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(dq_bytes / (dq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    per_kernel["attn_bwd_dkdv_kernel"]["bound"] = "mfma"
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
        "preprocess_ms": round(pre_ms, 4),
        "measured_peak": MFMA_MEASURED_TFLOPS[w.dtype],
        "frac_of_measured_peak": round(per_kernel[dom]["tflops"] / MFMA_MEASURED_TFLOPS[w.dtype], 4),
    }
    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("cpu baseline: timing the oracle backward on a bounded sample ...")
        cpu = cpu_baseline(w, inp, args.cpu_baseline_seconds)
    cfg = {"workload": w.name, "dtype": w.dtype, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
           "seqlen": (int(inp["lengths_q"].max()) if w.varlen else w.seqlen), "head_dim": w.head_dim,
           "causal": w.causal, "varlen": w.varlen, "deterministic": args.deterministic,
           "flop_per_step": flops, "parallelism": "single GPU"}
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, see workloads/)",
        "config": cfg,
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
