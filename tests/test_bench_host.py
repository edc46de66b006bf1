"""Host-side pieces of bench.py, on the CPU: the source digest that decides
whether the committed HBM-traffic counters still describe the kernels, the
committed counters' agreement with the committed sources, the CPU model
string, and the CPU-baseline leg on a small workload."""
import json
import os

import pytest
import torch

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) { /* block\n comment */ return x + 1; // line\n}\n"
    b = "int f(int x)\n{\n    return x + 1;\n}"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(b.replace("+ 1", "+ 2"))


def test_committed_traffic_counters_match_the_committed_sources():
    """Every entry of profiles/traffic.json was taken on the kernel sources as
    they stand (a kernel change must come with retaken counters; the bench
    reports traffic null otherwise)."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        doc = json.load(f)
    assert doc, "no traffic entries"
    for key, ent in doc.items():
        parts = key.split(":")
        config, path = parts[0], parts[1] if len(parts) > 1 else "kld"
        grad_dtype = parts[2] if len(parts) > 2 else "f32"
        assert bench.traffic_key(config, path, grad_dtype) == key
        assert ent["source_digest"] == bench.source_digest(path), f"{key}: counters taken on other sources"
        assert bench.recorded_traffic(config, path, grad_dtype) == ent["bytes_per_launch"]
        assert ent["bytes_per_launch"] == pytest.approx(ent["fetch_bytes"] + ent["write_bytes"])


def test_cpu_model_names_the_host():
    m = bench.cpu_model()
    assert isinstance(m, str) and m and m != "unknown"


def test_cpu_baseline_leg_on_a_small_workload():
    cfg = synth.CONFIGS["c1"]
    g = torch.Generator().manual_seed(0)
    base = (3 * torch.randn(cfg.n_rows, cfg.vocab, generator=g)).to(synth.torch_dtype(cfg.base_dtype))
    quant = (base.float() + 0.1 * torch.randn(cfg.n_rows, cfg.vocab, generator=g)).to(synth.torch_dtype(cfg.quant_dtype))
    out = bench.cpu_baseline(cfg, base, quant, 0.4, "kld")
    assert out["kind"] == "oracle" and out["unit"] == "rows/s" and out["value"] > 0
    assert out["cores"] >= 1 and out["host_cpus"] >= 1
    assert out["build"] in ("in-tree portable gcc -O3 -fopenmp (no -march)",
                            "gcc -O3 -march=native -fopenmp, compiled on this host at run time")
    other = [k for k in ("portable", "native") if k in out]
    assert len(other) <= 1
    for k in other:  # the slower build, beside the reported one
        assert 0 < out[k]["value"] <= out["value"]
    assert out["one_core"]["value"] > 0
    assert "rows" in out["sample"] and "of the same workload" in out["sample"]
