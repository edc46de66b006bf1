"""Calls whose grid exceeds what one launch may hold (the dispatch packet counts
work-items in 32 bits) are cut into pieces by the launchers. Every entry point
is run here on rows just past the first piece -- V = 8, so 8.4 million rows fit
in a few hundred MB -- with outputs pre-filled, so that a row no piece reached
shows; sampled rows around the piece boundary, at the ends and seeded others
are compared with the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import topk as otk
from tests.gpu_util import (assert_kl_close, compare_grad, compare_topk_compress, compare_topk_grad, grad_to_f64,
                            say, topk_kl_tol)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PIECE = (2 ** 31 - 1) // 256   # workgroups of 256 threads in one piece (the row launcher's bound too)
N = PIECE + 1000
V = 8
K = 3


@pytest.fixture(scope="module")
def rows():
    g = torch.Generator(device=DEV).manual_seed(20251203)
    b = (3.0 * torch.randn((N, V), generator=g, device=DEV)).to(torch.bfloat16)
    q = (b.float() + 0.3 * torch.randn((N, V), generator=g, device=DEV)).to(torch.bfloat16)
    torch.cuda.synchronize()
    yield b, q
    del b, q
    torch.cuda.empty_cache()


def _sample():
    r = np.concatenate([[0, 1, N - 2, N - 1], np.arange(PIECE - 3, PIECE + 3),
                        np.random.default_rng(5).integers(0, N, 18)])
    return np.unique(r)


def _take(t, rows):
    return t.index_select(0, torch.as_tensor(rows, device=t.device))


def test_rows_and_reductions_past_one_launch(rows):
    b, q = rows
    sel = _sample()
    kld = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    match = torch.full((N,), 255, dtype=torch.uint8, device=DEV)
    ab = torch.full((N,), -1, dtype=torch.int32, device=DEV)
    aq = torch.full((N,), -1, dtype=torch.int32, device=DEV)
    with qqe.Evaluator(V, N, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0, kld, match, ab, aq)
        s = ev.reduce(N)
        # one segment per row: more tiles and more segments than one launch holds
        offs = np.arange(N + 1, dtype=np.int64)
        ks = (qqe.kld_eval_summary * N)()
        lib = qqe.load_library()
        st = lib.kld_eval_reduce_segments(ev.handle, (ctypes.c_int64 * (N + 1)).from_buffer(offs), N, ks, None,
                                          None)
        assert st == qqe.KLD_OK, qqe.kld_eval_last_error()
        torch.cuda.synchronize()
    assert not torch.isnan(kld).any() and bool((match <= 1).all())
    assert bool(((ab >= 0) & (ab < V)).all()) and bool(((aq >= 0) & (aq < V)).all())
    m = match.cpu().numpy()
    assert s.n_rows == N and s.n_match == int(m.astype(np.int64).sum())
    o = oracle.rows(synth.to_numpy_bits(_take(b, sel)), synth.to_numpy_bits(_take(q, sel)))
    assert_kl_close(_take(kld, sel).cpu().numpy(), o.kl, "rows past one launch")
    assert np.array_equal(m[sel], o.match)
    assert np.array_equal(_take(ab, sel).cpu().numpy().astype(np.int64), o.argmax_base)
    assert np.array_equal(_take(aq, sel).cpu().numpy().astype(np.int64), o.argmax_quant)
    layout = np.dtype([("n_rows", "<i8"), ("kld_sum", "<f8"), ("kld_mean", "<f8"), ("kld_max", "<f8"),
                       ("kld_max_row", "<i8"), ("n_match", "<i8"), ("same_top1", "<f8")])
    assert layout.itemsize == ctypes.sizeof(qqe.kld_eval_summary)
    seg = np.frombuffer(memoryview(ks).cast("B"), dtype=layout)
    k64 = kld.cpu().numpy().astype(np.float64)
    assert (seg["n_rows"] == 1).all()
    assert np.array_equal(seg["kld_sum"], k64) and np.array_equal(seg["kld_max"], k64)
    assert np.array_equal(seg["kld_max_row"], np.arange(N)) and np.array_equal(seg["n_match"], m.astype(np.int64))
    say(f"[pieces] rows and both reduction levels over {N} rows / segments ok")


def test_dense_gradient_past_one_launch(rows):
    b, q = rows
    sel = _sample()
    out = torch.full((N, V), float("nan"), dtype=torch.float32, device=DEV)
    with qqe.Evaluator(V, N, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0)
        ev.grad(b, q, 0, 0.5, out, "f32")
        torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    nb, nq = synth.to_numpy_bits(_take(b, sel)), synth.to_numpy_bits(_take(q, sel))
    worst = compare_grad(grad_to_f64(_take(out, sel)), nb, nq, oracle.rows(nb, nq), 0.5, "f32",
                         ctx="gradient past one launch")
    say(f"[pieces] dense gradient over {N} rows ok (worst error / tolerance {worst:.3f})")
    del out
    torch.cuda.empty_cache()


def test_topk_paths_past_one_launch(rows):
    b, q = rows
    sel = _sample()
    idx = torch.full((N, K), -1, dtype=torch.int32, device=DEV)
    logp = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    rest = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    kl = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    match = torch.full((N,), 255, dtype=torch.uint8, device=DEV)
    out = torch.full((N, V), float("nan"), dtype=torch.float32, device=DEV)
    with qqe.Evaluator(V, N, "bf16", "bf16", device=DEV) as ev:
        s = torch.cuda.current_stream().cuda_stream
        qqe.kld_eval_topk_compress(ev.handle, b.data_ptr(), N, K, idx.data_ptr(), logp.data_ptr(), rest.data_ptr(),
                                   s)
        ev.rows_topk(idx, logp, rest, q, 0, kl, match)
        ev.grad_topk(idx, logp, q, 0, 1.0, out, "f32")
        torch.cuda.synchronize()
    assert bool(((idx >= 0) & (idx < V)).all()) and not torch.isnan(logp).any() and not torch.isnan(rest).any()
    assert not torch.isnan(kl).any() and bool((match <= 1).all()) and not torch.isnan(out).any()
    nb, nq = synth.to_numpy_bits(_take(b, sel)), synth.to_numpy_bits(_take(q, sel))
    lse_b = oracle.rows(nb, nb).lse_base
    lse_q = oracle.rows(nq, nq).lse_base
    gi, gl, gr = (_take(t, sel).cpu().numpy() for t in (idx, logp, rest))
    compare_topk_compress(gi, gl, gr, otk.compress(nb, K, lse_b), lse_b, ctx="compress past one launch")
    stored = otk.TopK(gi, gl, gr)
    o = otk.kl_topk(stored, nq, lse_q)
    g_kl = _take(kl, sel).cpu().numpy().astype(np.float64)
    tol = topk_kl_tol(o.kl)
    assert (np.abs(g_kl - o.kl) <= tol).all()
    assert np.array_equal(_take(match, sel).cpu().numpy(), o.match)
    worst = compare_topk_grad(grad_to_f64(_take(out, sel)), stored, nq, lse_q, 1.0, "f32",
                              ctx="top-K gradient past one launch")
    say(f"[pieces] compress, evaluate and top-K gradient over {N} rows ok (gradient worst {worst:.3f})")
    del out
    torch.cuda.empty_cache()


def test_read_probe_past_one_launch(rows):
    b, q = rows
    sink = qqe.read_probe(b, q)
    torch.cuda.synchronize()
    wb = b.view(torch.int32).cpu().numpy()
    wq = q.view(torch.int32).cpu().numpy()
    want = np.bitwise_xor.reduce(np.concatenate([wb, wq], axis=1), axis=1)
    assert np.array_equal(sink.cpu().numpy(), want)
    say(f"[pieces] read probe over {N} rows ok")

