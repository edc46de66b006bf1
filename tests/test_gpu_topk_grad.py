"""GPU parity of the gradient of the coarsened top-K KL with respect to the
quantized logits, against the float64 oracle, on the oracle's own stored form
(rounded to the float32 storage format, the same bytes on both sides)."""
import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import topk as otk
from tests.gpu_util import compare_topk_grad, grad_to_f64, qrest_rel_device, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _upload(t: otk.TopK):
    return (torch.as_tensor(np.ascontiguousarray(t.idx, np.int32), device=DEV),
            torch.as_tensor(np.ascontiguousarray(t.logp, np.float32), device=DEV),
            torch.as_tensor(np.ascontiguousarray(t.rest, np.float32), device=DEV))


def _stored(nb, k):
    return otk.to_storage(otk.compress(nb, k, oracle.rows(nb, nb).lse_base))


def _gpu_grad(stored, q, base_dtype, scale, dtype, row_offset=0, misalign=False):
    """rows_topk into handle rows [row_offset, row_offset + n), then grad_topk;
    with ``misalign`` the output starts two elements past a 16-byte boundary."""
    n, v = q.shape
    up = _upload(stored)
    want = torch.float32 if dtype == "f32" else torch.bfloat16
    with qqe.Evaluator(v, row_offset + max(n, 1), base_dtype, q.dtype, device=DEV) as ev:
        ev.rows_topk(*up, q, row_offset)
        if misalign:
            buf = torch.full((n * v + 8,), float("nan"), dtype=want, device=DEV)
            out = buf[2:2 + n * v].view(n, v)  # 8 bytes (f32) or 4 bytes (bf16) past the start
        else:
            out = torch.full((n, v), float("nan"), dtype=want, device=DEV)
        ev.grad_topk(up[0], up[1], q, row_offset, scale, out, dtype)
        torch.cuda.synchronize()
    return grad_to_f64(out)


CASES = [("c1", 24, 32000, 128), ("c2", 12, 151936, 128), ("c3", 8, 151936, 128), ("c4", 8, 262144, 128),
         ("c5", 12, 151936, 128), ("c2", 8, 151928, 1000), ("c4", 10, 4104, 7)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,n_rows,vocab,k", CASES)
def test_topk_grad_parity(name, n_rows, vocab, k, dtype):
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    stored = _stored(nb, k)
    scale = 1.0 / n_rows
    g = _gpu_grad(stored, q, cfg.base_dtype, scale, dtype, row_offset=3)
    worst = compare_topk_grad(g, stored, nq, oracle.rows(nq, nq).lse_base, scale, dtype, ctx=f"{name} k={k} {dtype}")
    say(f"[topk grad] {name} V={vocab} k={k} {dtype}: worst error/tolerance {worst:.3f}")


@pytest.mark.parametrize("vocab", [8701, 8704])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_grad_quant_rest_far_below_its_maximum(vocab, dtype):
    """float32 base rows around 3e4 against the same rows in bfloat16, whose
    values there are 128 apart: one planted token 20 above the rest rounds up
    to 30080 and everything else down to 29952, so each quant row puts all but
    ~1e-52 of its mass on that token (which the stored top-k holds) and its
    rest lies 128 nats below its maximum: R / Q_rest ~ 2^160 overflows
    float32 while every gradient entry stays small (a random case, seed
    201474, found such a row written as NaN). The unaligned vocabulary takes
    the element-wise path, the other the vector one."""
    g = np.random.default_rng(201474)
    n = 12
    zb = 3e4 + g.normal(0, 3, (n, vocab))
    zb[np.arange(n), g.integers(0, vocab, n)] = 3e4 + 20.0
    zq = zb + g.normal(0, 0.2, (n, vocab))
    b = torch.as_tensor(zb, dtype=torch.float32, device=DEV)
    q = torch.as_tensor(zq, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    lse_q = oracle.rows(nq, nq).lse_base
    for k in (128, 141):
        stored = _stored(nb, k)
        sel = np.zeros((n, vocab), bool)
        np.put_along_axis(sel, np.asarray(stored.idx, np.int64), True, axis=1)
        q_rest = np.where(sel, 0.0, np.exp(oracle.to_f64(nq) - lse_q[:, None])).sum(axis=1)
        R = np.asarray(stored.rest, np.float64)
        assert (R / q_rest > 2.0 ** 128).all() and (R > 1e-5).all(), "rows outside the intended class"
        gg = _gpu_grad(stored, q, "f32", 1.0 / n, dtype)
        assert np.isfinite(gg).all(), f"k={k} {dtype}: non-finite gradient entries"
        worst = compare_topk_grad(gg, stored, nq, lse_q, 1.0 / n, dtype, ctx=f"far quant rest V={vocab} k={k} {dtype}")
        say(f"[topk grad] far quant rest V={vocab} k={k} {dtype}: worst error/tolerance {worst:.3f}")


@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 8, 65, 513, 2056, 4104])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_topk_grad_edge_vocab_sizes_and_ties(vocab, dtypes):
    g0 = np.random.default_rng(vocab + 11)
    n = 5
    zb = np.round(g0.normal(0, 2.0, (n, vocab)), 1)
    zb[1] = 0.0
    zb[1, ::3] = -0.0
    zb[2] = 1.5
    zq = zb + np.round(g0.normal(0, 0.3, (n, vocab)), 2)
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtypes[1]), device=DEV)
    nb = synth.to_numpy_bits(torch.tensor(zb, dtype=synth.torch_dtype(dtypes[0])))
    nq = synth.to_numpy_bits(q)
    lse_q = oracle.rows(nq, nq).lse_base
    for k in sorted({1, min(vocab, 5), vocab if vocab <= 1024 else 1024}):
        stored = _stored(nb, k)
        for dtype in ("f32", "bf16"):
            g = _gpu_grad(stored, q, dtypes[0], -0.75, dtype)
            compare_topk_grad(g, stored, nq, lse_q, -0.75, dtype, ctx=f"V={vocab} k={k} {dtypes} -> {dtype}")
            if k == vocab and dtype == "f32":   # nothing coarsened: q - p of the full distribution
                qq = np.exp(oracle.to_f64(nq) - lse_q[:, None])
                pp = np.exp(oracle.to_f64(nb) - oracle.rows(nb, nb).lse_base[:, None])
                ref = -0.75 * (qq - pp)
                # q's log-space error, the float32 rounding of the stored log p
                assert np.all(np.abs(g - ref) <= 0.75 * (2e-5 * qq + 4e-6 * pp) + 2.0 ** -23 * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_grad_scalar_path_on_unaligned_output(dtype):
    """An output that is not 16-byte aligned takes the element-wise path."""
    cfg = synth.CONFIGS["c2"].scaled(n_rows=4, vocab=151936)
    b, q = synth.generate(cfg, device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    stored = _stored(nb, 128)
    g = _gpu_grad(stored, q, cfg.base_dtype, 2.0, dtype, misalign=True)
    compare_topk_grad(g, stored, nq, oracle.rows(nq, nq).lse_base, 2.0, dtype, ctx=f"unaligned {dtype}")


def test_topk_grad_bad_stored_indices_poison_only_their_row():
    cfg = synth.CONFIGS["c4"].scaled(n_rows=4, vocab=4104)
    b, q = synth.generate(cfg, device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    stored = _stored(nb, 16)
    good = otk.TopK(stored.idx[:1], stored.logp[:1], stored.rest[:1])
    stored.idx[1, 3] = stored.idx[1, 5]       # repeated id
    stored.idx[2, 0] = 4104                   # out of range
    stored.idx[3, 7] = -1                     # negative
    g = _gpu_grad(stored, q, "bf16", 1.0, "f32")
    assert np.all(np.isnan(g[1:]))
    compare_topk_grad(g[:1], good, nq[:1], oracle.rows(nq[:1], nq[:1]).lse_base, 1.0, "f32", ctx="good row")


def test_topk_grad_argument_errors():
    lib = qqe.load_library()
    with qqe.Evaluator(64, 4, "f32", "f32", device=DEV) as ev:
        z = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
        i = torch.zeros((4, 8), dtype=torch.int32, device=DEV)
        f = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
        p, ip, fp = z.data_ptr(), i.data_ptr(), f.data_ptr()
        for k in (0, 65, 1025, -3):
            assert lib.kld_eval_grad_topk(ev.handle, ip, fp, k, p, 4, 0, 1.0, p, 0, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad_topk(ev.handle, ip, fp, 8, p, 4, 1, 1.0, p, 0, None) == qqe.KLD_ERR_RANGE
        assert lib.kld_eval_grad_topk(ev.handle, ip, fp, 8, p, 4, 0, 1.0, p, 7, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad_topk(ev.handle, ip, fp, 8, p, 4, 0, float("inf"), p, 0,
                                      None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad_topk(ev.handle, ip, fp, 8, p, 4, 0, 1.0, None, 0, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_grad_topk(ev.handle, ip, fp, 8, p, 0, 0, 1.0, None, 0, None) == qqe.KLD_OK


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_c2_topk_grad_sampled_rows_and_row_sums(dtype):
    """8192 x 151936 bf16 with k = 128 in the launch shape the benchmark times:
    sampled rows against the oracle, and every row's sum against 0 (the exact
    gradient sums to scale ((P + R) sum q - P - R) = 0 for any stored values).
    On the GPU the quant probabilities sum to 1 within the log-normaliser's
    error (2e-5 relative here) and Q_rest matches their sum outside the stored
    tokens within the evaluator's bound; the output rounding adds at most a
    half-ulp of each entry."""
    cfg = synth.CONFIGS["c2"]
    b, q = synth.generate(cfg, device=DEV)
    n, v, k = cfg.n_rows, cfg.vocab, 128
    scale = 1.0 / n
    want = torch.float32 if dtype == "f32" else torch.bfloat16
    with qqe.Evaluator(v, n, "bf16", "bf16", device=DEV) as ev:
        idx, logp, rest = ev.topk_compress(b, k)
        ev.rows_topk(idx, logp, rest, q)
        out = torch.empty((n, v), dtype=want, device=DEV)
        ev.grad_topk(idx, logp, q, 0, scale, out, dtype)
        torch.cuda.synchronize()
    sums = out.sum(dim=1, dtype=torch.float64).cpu().numpy()
    abssum = out.abs().sum(dim=1, dtype=torch.float64).cpu().numpy()
    R = rest.double().cpu().numpy()
    rnd = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -24
    tol = rnd * abssum + scale * (2e-5 + R * (qrest_rel_device(q, idx) + 2e-5)) + 1e-9 * abssum
    assert np.all(np.abs(sums) <= tol), f"row sums: worst |sum| / tol {np.max(np.abs(sums) / tol):.3f}"
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(9).integers(0, n, 14)]))
    sel = torch.as_tensor(rows, device=DEV)
    stored = otk.TopK(idx.index_select(0, sel).cpu().numpy(), logp.index_select(0, sel).cpu().numpy(),
                      rest.index_select(0, sel).cpu().numpy())
    nq = synth.to_numpy_bits(q.index_select(0, sel))
    g = grad_to_f64(out.index_select(0, sel))
    worst = compare_topk_grad(g, stored, nq, oracle.rows(nq, nq).lse_base, scale, dtype, ctx=f"c2 full {dtype}")
    say(f"[topk grad] c2 full {dtype}: {rows.size} sampled rows, worst error/tolerance {worst:.3f}")
    del b, q, out
    torch.cuda.empty_cache()
