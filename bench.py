"""Throughput of the fused KLD + same-top-1 comparison on one MI355X.

A step is one pass of the whole hot path over one batch: the row kernel over
every row of the workload (per-token KLD, both argmaxes, match flag, both
log-normalisers) followed by the deterministic reduction to the summary
(mean / max KLD, match count), which the GPU writes into pinned host memory
(kld_eval_reduce_async: the host does not wait for each step's summary; it
synchronizes once at the end of the timed region and reads the last one).
The same steps with the host waiting for every summary (kld_eval_reduce) are
timed afterwards and reported as "blocking_reduce". Inputs are generated on
the GPU before the timed region and stay resident in HBM; the read ceiling of
the same buffers is measured before the warm-up steps. The row kernel and the
read probe are timed by HIP events that their launches record themselves
(kld_eval_rows_timed, kld_eval_read_probe), so that no marker packets sit
between the events and the kernel; the other paths use an event pair recorded
on the stream around each launch.

Default workload: one 8192-token context at a Qwen-class vocabulary,
8192 rows x V=151936, bf16 base vs bf16 quant (planted peaks, 2% moved).

Other paths (--path): "tokens" adds the next-token ids (same pass: per-token
log-probabilities, then the token summary as well); "grad" times the
gradient of the KL with respect to the quantized logits over every row (the
forward pass runs once before the timed region to save the normalisers);
"topk" times the coarsened KL of the full quant rows from the base rows stored
as their top-128 tokens + rest of mass (stored once before the timed region),
then the reduction; "compress" times storing the base rows in that form;
"topk_grad" times the gradient of that coarsened KL with respect to the
quantized logits (stored form and forward pass made once before the timed
region).

Prints one JSON line; see --help for options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# The arithmetic type of every kernel on the path: bfloat16 inputs are widened
# exactly to float32 and all per-element work is float32 (per-row and summary
# values float64). The input types are in config (base_dtype, quant_dtype).
COMPUTE_DTYPE = "f32"
METRIC = "logit rows/sec + HBM GB/s, fused KLD+top-1 match (V=151936, bf16, 1 GPU)"
METRICS = {
    "kld": METRIC,
    "tokens": "logit rows/sec + HBM GB/s, fused KLD+top-1 match + next-token log-probabilities (1 GPU)",
    "grad": "logit rows/sec + HBM GB/s, gradient of KL(base||quant) w.r.t. the quantized logits (1 GPU)",
    "topk": "logit rows/sec + HBM GB/s, coarsened KL of full quant rows from stored top-128 + rest base rows (1 GPU)",
    "compress": "logit rows/sec + HBM GB/s, base rows -> stored top-128 + rest of mass (1 GPU)",
    "topk_grad": "logit rows/sec + HBM GB/s, gradient of the coarsened top-128 KL w.r.t. the quantized logits "
                 "(1 GPU)",
}
KERNELS = {"kld": "kld_rows_kernel", "tokens": "kld_rows_kernel", "grad": "kld_grad_kernel",
           "topk": "topk_eval_kernel", "compress": "topk_compress_kernel", "topk_grad": "topk_grad_kernel"}
SOURCES = {"kld": ("kld_row.hip", "kld_kernels.h", "kld_bf16_pairs.h"),
           "tokens": ("kld_row.hip", "kld_kernels.h", "kld_bf16_pairs.h"),
           "grad": ("kld_grad.hip", "kld_kernels.h", "kld_bf16_pairs.h"),
           "topk": ("kld_topk.hip", "kld_kernels.h", "kld_bf16_pairs.h"),
           "compress": ("kld_topk.hip", "kld_kernels.h", "kld_bf16_pairs.h"),
           "topk_grad": ("kld_topk.hip", "kld_kernels.h", "kld_bf16_pairs.h")}
GRAD_PATHS = ("grad", "topk_grad")
TOPK = 128  # stored tokens per base row (the model card's top-128)
ROW_KERNEL = KERNELS["kld"]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps first (about 0.1 s on c2: enough for the clocks to settle)")
    p.add_argument("--config", default="c2", help="c1..c5 (c2 is the headline workload)")
    p.add_argument("--path", default="kld", choices=sorted(METRICS), help="which part of the path a step runs")
    p.add_argument("--grad-dtype", default="f32", choices=["f32", "bf16"], help="gradient output type (--path grad, topk_grad)")
    p.add_argument("--topk", type=int, default=TOPK,
                   help="stored tokens per base row for --path topk, compress, topk_grad (1..1024; default 128)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the CPU-baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="also run a plain elementwise copy of BYTES bytes (read BYTES, write BYTES) three "
                        "times; its HBM counters scale the counters of the row kernel")
    return p.parse_args()


def code_text(src: str) -> str:
    """C++ source with comments removed and whitespace collapsed: edits to
    comments or layout leave the kernels, and so the digest, unchanged."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_digest(path: str = "kld") -> str:
    h = hashlib.sha256()
    for f in SOURCES[path]:
        with open(os.path.join(ROOT, "quantization_quality_eval_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_key(config: str, path: str, grad_dtype: str = "f32") -> str:
    if path == "kld":
        return config
    return f"{config}:{path}" + (f":{grad_dtype}" if path in GRAD_PATHS else "")


def recorded_traffic(config: str, path: str = "kld", grad_dtype: str = "f32"):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source; otherwise None."""
    fn = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(fn) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    ent = doc.get(traffic_key(config, path, grad_dtype))
    if not ent or ent.get("source_digest") != source_digest(path):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(cfg, base, quant, budget_s: float, path: str = "kld", tokens=None):
    """The oracle timed on this host's cores over the rows of the same
    workload, in order and wrapping around to the first row until each leg's
    share of the time budget is spent: the in-tree portable build and a copy
    of the same C source compiled here with -march=native (the faster of the
    two is the reported value, the other is kept beside it), then the faster
    build on one core."""
    import tempfile

    import numpy as np

    import oracle
    import synth
    from oracle import grad as ograd
    from oracle import tokens as otok
    from oracle import topk as otk_
    from oracle.build import build_oracle

    n = cfg.n_rows
    batch = {"grad": 8, "topk": 8, "compress": 8, "topk_grad": 8}.get(path, 64)
    threads = oracle.max_threads()
    what = {"kld": "float64 C oracle, OpenMP over rows",
            "tokens": "float64 C oracle (OpenMP over rows) + NumPy next-token log-probabilities",
            "grad": "float64 C oracle for the normalisers (OpenMP over rows) + NumPy float64 gradient",
            "topk": "float64 C oracle for the normalisers + NumPy top-128 selection and coarsened KL",
            "compress": "float64 C oracle for the normaliser + NumPy top-128 selection",
            "topk_grad": "float64 C oracle for the normalisers + NumPy float64 gradient of the coarsened KL "
                         "(stored top-128 form made outside the timed part)"}[path]

    def timed(lib, budget, n_threads=0, batch_rows=batch):
        done, spent = 0, 0.0
        while spent < budget:
            r0 = done % n
            r1 = min(n, r0 + batch_rows)
            nb = synth.to_numpy_bits(base[r0:r1])
            nq = synth.to_numpy_bits(quant[r0:r1])
            if path == "topk_grad":
                st = otk_.to_storage(otk_.compress(nb, TOPK, oracle.rows(nb, nb, lib=lib).lse_base))
            t0 = time.perf_counter()
            o = oracle.rows(nb, nq, n_threads=n_threads, lib=lib)
            if n_threads == 1:
                pass  # one core: normalisers and KL only
            elif path == "tokens":
                otok.token_rows(nb, nq, tokens[r0:r1], o.lse_base, o.lse_quant)
            elif path == "grad":
                ograd.grad_rows(nb, nq, o.lse_base, o.lse_quant, 1.0 / n)
            elif path in ("topk", "compress"):
                t = otk_.compress(nb, TOPK, o.lse_base)
                if path == "topk":
                    otk_.kl_topk(otk_.to_storage(t), nq, o.lse_quant)
            elif path == "topk_grad":
                otk_.grad_topk(st, nq, o.lse_quant, 1.0 / n)
            spent += time.perf_counter() - t0
            done += r1 - r0
        return done, spent

    def rows_taken(done):
        return f"first {done} of {n} rows" if done <= n else f"{done} rows ({done / n:.1f} passes over the {n})"

    def leg(lib, build):
        done, spent = timed(lib, budget_s / 2)
        return {"lib": lib, "value": done / spent, "unit": "rows/s", "cores": threads, "build": build,
                "rows": rows_taken(done), "seconds": spent}

    legs = {"portable": leg(None, "in-tree portable gcc -O3 -fopenmp (no -march)")}
    try:
        native_path = os.path.join(tempfile.mkdtemp(prefix="kldoracle-"), "libkldoracle_native.so")
        nlib = oracle.open_library(build_oracle(native=True, out=native_path))
        legs["native"] = leg(nlib, "gcc -O3 -march=native -fopenmp, compiled on this host at run time")
    except Exception as exc:  # no compiler on this host: report the portable build only
        print(f"[bench] native oracle build failed ({exc}); reporting the portable build", file=sys.stderr)
    best_key = max(legs, key=lambda k: legs[k]["value"])
    best = legs[best_key]
    done1, spent1 = timed(best["lib"], budget_s / 4, n_threads=1, batch_rows=8)
    oracle.max_threads(threads)
    out = {"value": best["value"], "unit": "rows/s", "cores": threads, "kind": "oracle", "build": best["build"],
           "sample": f"{best['rows']} of the same workload, {what} ({best['seconds']:.1f} s)",
           "gb_per_s": best["value"] * cfg.bytes_per_row / 1e9,
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    for k, o in legs.items():
        if k != best_key:  # the slower build, beside the reported one
            out[k] = {"value": o["value"], "unit": "rows/s", "cores": threads, "build": o["build"],
                      "sample": f"{o['rows']} ({o['seconds']:.1f} s)"}
    out["one_core"] = {"value": done1 / spent1, "unit": "rows/s", "kind": "oracle, normalisers and KL only",
                       "build": best["build"], "sample": f"{rows_taken(done1)} ({spent1:.1f} s)"}
    return out


def cpu_model() -> str:
    """The CPU model as lscpu names it, with its family / model / stepping
    numbers (a virtual machine may report only a generic name), falling back
    to /proc/cpuinfo."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        fields = {}
        for line in out.splitlines():
            key, sep, val = line.partition(":")
            if sep and key.strip() not in fields:
                fields[key.strip()] = val.strip()
        if "Model name" in fields:
            ids = ", ".join(f"{k.lower()} {fields[k]}" for k in ("CPU family", "Model", "Stepping") if k in fields)
            return fields["Model name"] + (f" ({ids})" if ids else "")
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


READ_ONLY = ("kld", "tokens", "topk", "compress")  # paths whose large streams are reads only


def read_ceiling(qqe, path, base, quant, step_rows, n_chunks, stream, reps=10):
    """The read probe over the same buffers the path streams (both rows, the
    quant rows or the base rows), launched per chunk like the path, in both
    of its shapes (one and four waves per row): the faster shape's rate is
    the attainable read rate the path's kernel is set against. Rows of
    different widths (an f32 side and a bf16 side) are read by two launches,
    one per buffer, inside the same timed bracket."""
    import torch
    arrays = {"kld": (base, quant), "tokens": (base, quant), "topk": (quant, None), "compress": (base, None)}[path]
    bytes_per_launch = sum(x[:step_rows].numel() * x.element_size() for x in arrays if x is not None)
    shapes = {}
    # timed like the path's kernel: the probe's launches record the events
    # themselves (the first one start, the last one stop); a first record
    # creates the events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    e1.record(stream)
    e1.synchronize()
    for waves in (1, 4):
        times = []
        for rep in range(reps + 3):
            for i in range(n_chunks):
                sl = slice(i * step_rows, (i + 1) * step_rows)
                a, b = arrays
                with torch.cuda.stream(stream):
                    if b is not None and b.dtype != a.dtype:
                        qqe.read_probe(a[sl], None, stream=stream, waves_per_row=waves, start_event=e0)
                        qqe.read_probe(b[sl], None, stream=stream, waves_per_row=waves, stop_event=e1)
                    else:
                        qqe.read_probe(a[sl], None if b is None else b[sl], stream=stream, waves_per_row=waves,
                                       start_event=e0, stop_event=e1)
                e1.synchronize()
                if rep >= 3:
                    times.append(e0.elapsed_time(e1))
        shapes[waves] = (statistics.median(times), min(times))
    waves = min(shapes, key=lambda w: shapes[w][0])
    med, best = shapes[waves]
    return {"kernel": "kld_read_probe_kernel", "bytes_per_launch": bytes_per_launch, "waves_per_row": waves,
            "median_ms": med, "best_ms": best, "gb_per_s": bytes_per_launch / (med * 1e-3) / 1e9,
            "best_gb_per_s": bytes_per_launch / (best * 1e-3) / 1e9,
            "by_shape_gb_per_s": {f"{w} wave{'s' if w > 1 else ''} per row": bytes_per_launch / (t[0] * 1e-3) / 1e9
                                  for w, t in shapes.items()}}


def main():
    global TOPK
    args = parse()
    TOPK = args.topk
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(rows are independent: several GPUs would each run this kernel on their own row range).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import quantization_quality_eval_amd as qqe
    import synth
    from quantization_quality_eval_amd import kld_eval_topk_compress

    qqe.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    n, v = cfg.n_rows, cfg.vocab
    if not 1 <= TOPK <= min(1024, v):
        print(f"--topk must be in [1, {min(1024, v)}]", file=sys.stderr)
        sys.exit(2)
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
    kernel_ms = []
    span_ms = []  # per step: first chunk launch's start to the last one's end (chunks may overlap)
    path = args.path
    tokens_host = synth.tokens(cfg, plan=plan) if path == "tokens" else None
    tok = torch.as_tensor(tokens_host, device=dev) if tokens_host is not None else None
    grad_size = 4 if args.grad_dtype == "f32" else 2
    grads = []
    stored = []
    if path in ("topk", "compress", "topk_grad"):
        # the base rows in stored form, per chunk (made once; "compress" remakes them each step)
        for i in range(n_chunks):
            stored.append(ev.topk_compress(base[i * step_rows:(i + 1) * step_rows], TOPK))
        torch.cuda.synchronize()
    if path == "grad":
        # forward once (saves the normalisers); one output buffer per stream
        for i in range(n_chunks):
            ev.rows(base[i * step_rows:(i + 1) * step_rows], quant[i * step_rows:(i + 1) * step_rows],
                    i * step_rows)
        gdt = torch.float32 if args.grad_dtype == "f32" else torch.bfloat16
        grads = [torch.empty((step_rows, v), dtype=gdt, device=dev) for _ in streams]
        torch.cuda.synchronize()
    if path == "topk_grad":
        # forward once (saves the quant normalisers and rest masses); one output buffer per stream
        for i in range(n_chunks):
            ev.rows_topk(*stored[i], quant[i * step_rows:(i + 1) * step_rows], i * step_rows)
        gdt = torch.float32 if args.grad_dtype == "f32" else torch.bfloat16
        grads = [torch.empty((step_rows, v), dtype=gdt, device=dev) for _ in streams]
        torch.cuda.synchronize()

    def launch(i, s, mark=None):
        sl = slice(i * step_rows, (i + 1) * step_rows)
        if path == "grad":
            ev.grad(base[sl], quant[sl], i * step_rows, 1.0 / n, out=grads[i % len(streams)],
                    dtype=args.grad_dtype, stream=s)
        elif path == "topk":
            ev.rows_topk(*stored[i], quant[sl], i * step_rows, stream=s)
        elif path == "topk_grad":
            ev.grad_topk(stored[i][0], stored[i][1], quant[sl], i * step_rows, 1.0 / n,
                         out=grads[i % len(streams)], dtype=args.grad_dtype, stream=s)
        elif path == "compress":
            idx, logp, rest = stored[i]
            kld_eval_topk_compress(ev.handle, base[sl].data_ptr(), step_rows, TOPK, idx.data_ptr(), logp.data_ptr(),
                                   rest.data_ptr(), s.cuda_stream)
        elif path == "kld" and mark is not None:
            # the row kernel's launch records the step's timing events itself
            ev.rows(base[sl], quant[sl], i * step_rows, stream=s, start_event=mark[0], stop_event=mark[1])
        else:
            ev.rows(base[sl], quant[sl], i * step_rows, stream=s, tokens=None if tok is None else tok[sl])

    ASYNC_REDUCE = ("kld", "topk")  # paths whose step ends with the KLD summary alone
    TIMED_BY_LAUNCH = ("kld",)  # paths whose kernel launch records the timing events (no marker packets)
    summary_buf = torch.empty(64, dtype=torch.uint8, pin_memory=True)

    def step(marks=None, blocking=False):
        """One pass over every chunk, then the reduction. With ``marks`` (a list
        of (start, stop) event pairs per chunk) the chunk launches are timed.
        The reduction of the kld and topk paths is enqueued without a host wait
        (kld_eval_reduce_async: the GPU writes the summary into pinned host
        memory) unless ``blocking``; the tokens path waits for both summaries."""
        for s in streams:
            if s is not main_stream:
                s.wait_stream(main_stream)
        for i in range(n_chunks):
            s = streams[i % len(streams)]
            with torch.cuda.stream(s):
                if marks is not None and path not in TIMED_BY_LAUNCH:
                    marks[i][0].record(s)
                launch(i, s, None if marks is None else marks[i])
                if marks is not None and path not in TIMED_BY_LAUNCH:
                    marks[i][1].record(s)
        summ = tsum = None
        if path in ("grad", "compress", "topk_grad"):
            for s in streams:
                if s is not main_stream:
                    main_stream.wait_stream(s)
        elif path in ASYNC_REDUCE and not blocking:
            ev.reduce_async(n, out=summary_buf, stream=main_stream)
        else:
            summ = ev.reduce(n, stream=main_stream)
            if path == "tokens":
                tsum = ev.reduce_tokens(n, stream=main_stream)
        return summ, tsum

    # the read ceiling of the same buffers first: it calibrates the roofline
    # figure and streams the same bytes before the warm-up steps
    ceiling = (read_ceiling(qqe, path, base, quant, step_rows, n_chunks, main_stream, reps=30)
               if path in READ_ONLY else None)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_chunks)]
             for _ in range(args.steps)]
    if path in TIMED_BY_LAUNCH:
        # a first record creates each event, outside the timed region
        for m in marks:
            for a, b in m:
                a.record(main_stream)
                b.record(main_stream)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        summ, tsum = step(marks[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for m in marks:
        kernel_ms.extend(a.elapsed_time(b) for a, b in m)
        if n_chunks > 1:
            span_ms.append(max(m[0][0].elapsed_time(b) for _, b in m))
    ks = [f"{t:.4f}" for t in kernel_ms]
    print(f"[bench] {KERNELS[path]} ms per launch, first: {' '.join(ks[:6])}; last: {' '.join(ks[-6:])}",
          file=sys.stderr, flush=True)
    blocking = None
    if path in ASYNC_REDUCE:
        summ = qqe.summary_from_bytes(summary_buf)
        # the same steps with the host waiting for every summary (kld_eval_reduce)
        t1 = time.perf_counter()
        for _ in range(args.steps):
            bsum, _ = step(blocking=True)
        torch.cuda.synchronize()
        wall_b = time.perf_counter() - t1
        assert bsum == summ, f"asynchronous summary {summ} differs from the blocking one {bsum}"
        blocking = {"ms_per_step": wall_b * 1e3 / args.steps, "value": n * args.steps / wall_b,
                    "reduce": "kld_eval_reduce (the host waits for each summary)"}
    if path in ("grad", "compress", "topk_grad"):
        if path == "compress":
            for i in range(n_chunks):
                ev.rows_topk(*stored[i], quant[i * step_rows:(i + 1) * step_rows], i * step_rows)
        summ = ev.reduce(n)
    ev.close()
    del grads

    stored_bytes = TOPK * 8 + 4
    row_bytes = {"grad": cfg.bytes_per_row + v * grad_size,
                 "topk": v * synth._size(cfg.quant_dtype) + stored_bytes,
                 "compress": v * synth._size(cfg.base_dtype) + stored_bytes,
                 "topk_grad": v * synth._size(cfg.quant_dtype) + TOPK * 8 + v * grad_size}.get(
                     path, cfg.bytes_per_row)
    ms_per_step = wall * 1e3 / args.steps
    rows_per_s = n * args.steps / wall
    bytes_per_launch = step_rows * row_bytes
    avg_kernel_ms = sum(kernel_ms) / len(kernel_ms)
    achieved = bytes_per_launch / (avg_kernel_ms * 1e-3) / 1e9
    # the counters were taken with the default top-K width
    traffic = (recorded_traffic(args.config, path, args.grad_dtype)
               if path not in ("topk", "compress", "topk_grad") or TOPK == 128 else None)
    workload = (f"{args.config}: {n} rows x V={v}, base {cfg.base_dtype} vs quant {cfg.quant_dtype}, "
                f"{cfg.kind} recipe" + (f", {n_chunks} chunks of {step_rows} rows on "
                                        f"{len(streams)} streams" if n_chunks > 1 else ""))
    if path == "tokens":
        workload += ", with next-token ids"
    if path in GRAD_PATHS:
        workload += f", gradient written as {args.grad_dtype}"
    if path == "topk":
        workload += f", base stored as top-{TOPK} + rest of mass (quant rows in full)"
    if path == "compress":
        workload += f", base rows stored as top-{TOPK} + rest of mass"
    if path == "topk_grad":
        workload += f", base stored as top-{TOPK} + rest of mass"
    out = {
        "metric": METRICS[path],
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": COMPUTE_DTYPE,
        "data": "synthetic",
        "gb_per_s": rows_per_s * row_bytes / 1e9,
        "config": {
            "workload": workload,
            "rows": n, "vocab": v, "base_dtype": cfg.base_dtype, "quant_dtype": cfg.quant_dtype,
            "input_bytes": cfg.total_bytes, "path": path,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": KERNELS[path],
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "avg_kernel_ms": avg_kernel_ms,
            "median_kernel_ms": statistics.median(kernel_ms),
            "best_kernel_ms": min(kernel_ms),
            "read_ceiling": ceiling,
            "frac_of_read_ceiling": None if ceiling is None else achieved / ceiling["gb_per_s"],
        },
        "summary": {"kld_mean": summ.kld_mean, "kld_max": summ.kld_max, "kld_max_row": summ.kld_max_row,
                    "same_top1": summ.same_top1},
    }
    if blocking is not None:
        out["blocking_reduce"] = blocking
    if span_ms:
        # chunks on several streams overlap, so a launch's own rate counts one
        # of the kernels in flight: the whole step's chunk launches, start of
        # the first to end of the last, give the aggregate
        span = statistics.median(span_ms)
        agg = n_chunks * bytes_per_launch / (span * 1e-3) / 1e9
        out["roofline"]["aggregate"] = {"chunks": n_chunks, "streams": len(streams), "median_span_ms": span,
                                        "gb_per_s": agg, "frac": agg / HBM_PEAK_GBS,
                                        # the probe reads one chunk per launch, one launch at a time
                                        "frac_of_read_ceiling": None if ceiling is None else agg / ceiling["gb_per_s"]}
    if tsum is not None:
        out["token_summary"] = {"n_scored": tsum.n_scored, "ppl_base": tsum.ppl_base, "ppl_quant": tsum.ppl_quant,
                                "ppl_ratio": tsum.ppl_ratio, "dp_mean": tsum.dp_mean, "dp_rms": tsum.dp_rms}
    if path in GRAD_PATHS:
        out["config"]["grad_dtype"] = args.grad_dtype
    if path in ("topk", "compress", "topk_grad"):
        out["config"]["topk"] = TOPK
        if path == "compress":
            out["roofline"]["note"] = ("algorithmic bytes = one read of the base rows + the stored form written; "
                                       "the sampled bound reads every 4th step of each row before the full pass "
                                       "(1.25 reads per row, k <= 256)")
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, base, quant, args.cpu_seconds, path, tokens_host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
