"""GPU parity of the gradient of the per-token KL with respect to the quantized
logits (scale * (q - p)), against the float64 oracle, element by element.

Oracle-sized cases compare every element; the full-size headline workload is
run in the launch configuration the benchmark times and checked on sampled
rows element by element and on every row through a property that holds at any
size (each gradient row sums to zero, within the bound its elements' bounds
give).
"""
import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from tests.gpu_util import LSE_REL, compare_grad, grad_to_f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _forward_and_grad(b, q, scale, out_dtype, row_offset=0, ev=None):
    n = b.shape[0]
    own = ev is None
    if own:
        ev = qqe.Evaluator(b.shape[1], n + row_offset, b.dtype, q.dtype, device=DEV)
    ev.rows(b, q, row_offset)
    g = ev.grad(b, q, row_offset, scale, dtype=out_dtype)
    torch.cuda.synchronize()
    if own:
        ev.close()
    return g


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,n_rows,vocab", [
    ("c1", 64, 32000),
    ("c2", 24, 151936),
    ("c3", 16, 151936),
    ("c4", 16, 262144),
    ("c5", 24, 151936),
    ("c2", 20, 151928),
    ("c4", 20, 4104),
])
def test_grad_parity_oracle_sized(name, n_rows, vocab, out_dtype):
    say(f"[grad] {name} n={n_rows} V={vocab} -> {out_dtype}")
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    scale = 1.0 / n_rows
    g = _forward_and_grad(b, q, scale, out_dtype)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    o = oracle.rows(nb, nq)
    worst = compare_grad(grad_to_f64(g), nb, nq, o, scale, out_dtype, ctx=f"{name} {out_dtype}")
    say(f"[grad] {name} {out_dtype}: worst error / tolerance {worst:.3f}")


@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 8, 65, 511, 4096 + 8, 8192 + 3])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_grad_edge_vocab_sizes(vocab, dtypes):
    g0 = np.random.default_rng(vocab + 11)
    n = 9
    zb = torch.tensor(g0.normal(0, 3.0, (n, vocab)), dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    zq = (zb.float() + torch.tensor(g0.normal(0, 0.5, (n, vocab)), dtype=torch.float32, device=DEV)).to(
        synth.torch_dtype(dtypes[1]))
    for out_dtype, scale in (("f32", 1.0), ("bf16", -2.5)):
        g = _forward_and_grad(zb, zq, scale, out_dtype)
        nb, nq = synth.to_numpy_bits(zb), synth.to_numpy_bits(zq)
        compare_grad(grad_to_f64(g), nb, nq, oracle.rows(nb, nq), scale, out_dtype, ctx=f"V={vocab} {dtypes}")
        if vocab == 1:
            assert torch.all(g == 0)


def test_grad_identical_rows_and_row_offsets():
    cfg = synth.CONFIGS["c5"].scaled(n_rows=30, vocab=151936)
    b, _ = synth.generate(cfg, device=DEV)
    with qqe.Evaluator(cfg.vocab, 40, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, b, 10)
        g = ev.grad(b, b, 10, 1.0)
        torch.cuda.synchronize()
        assert torch.all(g == 0)
    # rows evaluated at an offset and in pieces give the same gradient as one call
    b, q = synth.generate(cfg, device=DEV)
    whole = _forward_and_grad(b, q, 0.5, "f32")
    with qqe.Evaluator(cfg.vocab, 40, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b[:13], q[:13], 7)
        ev.rows(b[13:], q[13:], 20)
        g1 = ev.grad(b[:13], q[:13], 7, 0.5)
        g2 = ev.grad(b[13:], q[13:], 20, 0.5)
        torch.cuda.synchronize()
    assert torch.equal(torch.cat([g1, g2]), whole)


def test_grad_unaligned_and_guard_bands():
    cfg = synth.CONFIGS["c1"].scaled(n_rows=6, vocab=4096)
    b, q = synth.generate(cfg, device=DEV)
    n, v = b.shape
    vb = torch.empty(n * v + 1, dtype=b.dtype, device=DEV)[1:].view(n, v)
    vb.copy_(b)
    out = torch.full((n * v + 64,), 7.0, dtype=torch.float32, device=DEV)
    with qqe.Evaluator(v, n, "f32", "f32", device=DEV) as ev:
        ev.rows(vb, q, 0)
        ev.grad(vb, q, 0, 1.0, out=out[1:1 + n * v])            # unaligned input and output: element path
        ref = ev.grad(b, q, 0, 1.0)                             # aligned: vector path
        torch.cuda.synchronize()
    assert out[0].item() == 7.0 and torch.all(out[1 + n * v:] == 7.0)
    assert torch.equal(out[1:1 + n * v].view(n, v), ref)


def test_grad_argument_errors():
    with qqe.Evaluator(64, 4, "f32", "f32", device=DEV) as ev:
        z = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
        ev.rows(z, z, 0)
        lib = qqe.load_library()
        out = torch.empty((4, 64), dtype=torch.float32, device=DEV)
        p, o = z.data_ptr(), out.data_ptr()
        assert lib.kld_eval_grad(ev.handle, p, p, 4, 0, 1.0, o, 2, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad(ev.handle, p, p, 4, 0, float("nan"), o, 0, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad(ev.handle, p, p, 4, 0, 1.0, None, 0, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad(ev.handle, p, p, 4, 1, 1.0, o, 0, None) == qqe.KLD_ERR_RANGE
        assert lib.kld_eval_grad(ev.handle, p, p, -1, 0, 1.0, o, 0, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad(ev.handle, p, p, 0, 0, 1.0, None, 0, None) == qqe.KLD_OK


@pytest.mark.slow
def test_full_c2_grad_sampled_rows_and_row_sums():
    cfg = synth.CONFIGS["c2"]
    b, q = synth.generate(cfg, device=DEV)
    n, v = b.shape
    scale = 1.0 / n
    plan = synth.row_plan(cfg)
    with qqe.Evaluator(v, n, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0)
        g = ev.grad(b, q, 0, scale)
        lse_b = torch.empty(n, dtype=torch.float32, device=DEV)
        lse_q = torch.empty(n, dtype=torch.float32, device=DEV)
        ev.copy_lse(0, n, lse_b, lse_q)
        torch.cuda.synchronize()
    # every row: the gradient sums to zero within the sum of its elements' bounds
    row_sum = g.double().sum(dim=1).cpu().numpy()
    abs_sum = g.double().abs().sum(dim=1).cpu().numpy()
    zmax_b = b.float().max(dim=1).values.double().cpu().numpy()
    zmin_b = b.float().min(dim=1).values.double().cpu().numpy()
    zmin_q = q.float().min(dim=1).values.double().cpu().numpy()
    zmax_q = q.float().max(dim=1).values.double().cpu().numpy()
    lb, lq = lse_b.double().cpu().numpy(), lse_q.double().cpu().numpy()
    span_b = np.maximum(np.abs(zmax_b - lb), np.abs(zmin_b - lb)) + 1.0
    span_q = np.maximum(np.abs(zmax_q - lq), np.abs(zmin_q - lq)) + 1.0
    lse_tol = (LSE_REL * np.maximum(np.abs(lb), 1) + 1e-6) + (LSE_REL * np.maximum(np.abs(lq), 1) + 1e-6)
    bound = scale * (lse_tol + 2.0 ** -23 * (span_b + span_q)) + 2.0 ** -22 * abs_sum
    assert np.all(np.abs(row_sum) <= bound), f"row sums: worst {np.max(np.abs(row_sum) / bound):.3f} of bound"
    # sampled rows, element by element: ends, moved-peak rows, seeded others
    moved = np.nonzero(plan.moved)[0]
    rows = np.unique(np.concatenate([[0, 1, n - 1], moved[:8], np.random.default_rng(3).integers(0, n, 21)]))
    idx = torch.as_tensor(rows, device=DEV)
    nb = synth.to_numpy_bits(b.index_select(0, idx))
    nq = synth.to_numpy_bits(q.index_select(0, idx))
    o = oracle.rows(nb, nq)
    worst = compare_grad(grad_to_f64(g.index_select(0, idx)), nb, nq, o, scale, "f32", ctx="c2 full, sampled rows")
    say(f"[grad] c2 full: {rows.size} sampled rows ok (worst error / tolerance {worst:.3f}); all row sums in bound")
    del g, b, q
    torch.cuda.empty_cache()
