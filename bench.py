"""Throughput of the fused KLD + same-top-1 comparison on one MI355X.

A step is one pass of the whole hot path over one batch: the row kernel over
every row of the workload (per-token KLD, both argmaxes, match flag, both
log-normalisers) followed by the deterministic reduction to the summary
(mean / max KLD, match count), which returns to the host. Inputs are
generated on the GPU before the timed region and stay resident in HBM.

Default workload: one 8192-token context at a Qwen-class vocabulary,
8192 rows x V=151936, bf16 base vs bf16 quant (planted peaks, 2% moved).

Prints one JSON line; see --help for options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "logit rows/sec + HBM GB/s, fused KLD+top-1 match (V=151936, bf16, 1 GPU)"
ROW_KERNEL = "kld_rows_kernel"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="c2", help="c1..c5 (c2 is the headline workload)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the CPU-baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="also run a plain elementwise copy of BYTES bytes (read BYTES, write BYTES) three "
                        "times; its HBM counters scale the counters of the row kernel")
    return p.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("kld_row.hip", "kld_kernels.h"):
        with open(os.path.join(ROOT, "quantization_quality_eval_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(config: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    ent = doc.get(config)
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(cfg, base, quant, budget_s: float):
    import numpy as np

    import oracle
    import synth

    n = cfg.n_rows
    batch = 64
    done, spent = 0, 0.0
    threads = oracle.max_threads()
    while done < n and spent < budget_s:
        r1 = min(n, done + batch)
        nb = synth.to_numpy_bits(base[done:r1])
        nq = synth.to_numpy_bits(quant[done:r1])
        t0 = time.perf_counter()
        oracle.rows(nb, nq)
        spent += time.perf_counter() - t0
        done = r1
    rows_s = done / spent
    return {"value": rows_s, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"first {done} of {n} rows of the same workload, float64 C oracle, OpenMP over rows "
                      f"({spent:.1f} s)",
            "gb_per_s": rows_s * cfg.bytes_per_row / 1e9,
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(rows are independent: several GPUs would each run this kernel on their own row range).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import quantization_quality_eval_amd as qqe
    import synth

    qqe.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    n, v = cfg.n_rows, cfg.vocab
    step_rows = cfg.chunk_rows or n
    n_chunks = n // step_rows
    print(f"[bench] generating {args.config}: {n} x {v} {cfg.base_dtype}/{cfg.quant_dtype} "
          f"({cfg.total_bytes / 1e9:.2f} GB)", file=sys.stderr, flush=True)
    base = torch.empty((n, v), dtype=synth.torch_dtype(cfg.base_dtype), device=dev)
    quant = torch.empty((n, v), dtype=synth.torch_dtype(cfg.quant_dtype), device=dev)
    plan = synth.row_plan(cfg)
    for i in range(n_chunks):
        synth.fill(cfg, base[i * step_rows:(i + 1) * step_rows], quant[i * step_rows:(i + 1) * step_rows],
                   i * step_rows, plan)
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copy: 3 x {args.calibrate_copy} bytes read + written", file=sys.stderr,
              flush=True)

    ev = qqe.Evaluator(v, n, cfg.base_dtype, cfg.quant_dtype, device=dev)
    main_stream = torch.cuda.current_stream(dev)
    streams = [main_stream] if cfg.streams <= 1 else [torch.cuda.Stream(device=dev) for _ in range(cfg.streams)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_chunks)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(n_chunks)]
    kernel_ms = []

    def step(record: bool):
        for s in streams:
            if s is not main_stream:
                s.wait_stream(main_stream)
        for i in range(n_chunks):
            s = streams[i % len(streams)]
            sl = slice(i * step_rows, (i + 1) * step_rows)
            with torch.cuda.stream(s):
                if record:
                    starts[i].record(s)
                ev.rows(base[sl], quant[sl], i * step_rows, stream=s)
                if record:
                    stops[i].record(s)
        summ = ev.reduce(n, stream=main_stream)
        if record:
            kernel_ms.extend(starts[i].elapsed_time(stops[i]) for i in range(n_chunks))
        return summ

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        summ = step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev.close()

    ms_per_step = wall * 1e3 / args.steps
    rows_per_s = n * args.steps / wall
    bytes_per_launch = step_rows * cfg.bytes_per_row
    avg_kernel_ms = sum(kernel_ms) / len(kernel_ms)
    achieved = bytes_per_launch / (avg_kernel_ms * 1e-3) / 1e9
    traffic = recorded_traffic(args.config)
    out = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "gb_per_s": rows_per_s * cfg.bytes_per_row / 1e9,
        "config": {
            "workload": f"{args.config}: {n} rows x V={v}, base {cfg.base_dtype} vs quant {cfg.quant_dtype}, "
                        f"{cfg.kind} recipe" + (f", {n_chunks} chunks of {step_rows} rows on "
                                                f"{len(streams)} streams" if n_chunks > 1 else ""),
            "rows": n, "vocab": v, "base_dtype": cfg.base_dtype, "quant_dtype": cfg.quant_dtype,
            "input_bytes": cfg.total_bytes,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ROW_KERNEL,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "avg_kernel_ms": avg_kernel_ms,
        },
        "summary": {"kld_mean": summ.kld_mean, "kld_max": summ.kld_max, "kld_max_row": summ.kld_max_row,
                    "same_top1": summ.same_top1},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, base, quant, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
