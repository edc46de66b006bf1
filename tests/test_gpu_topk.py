"""GPU parity of the top-K + rest-of-mass path: the compressor (base rows ->
stored form) and the evaluator (stored base rows + full quantized rows ->
coarsened KL, top-1 match), against the float64 oracle.

The evaluator is checked on the oracle's own stored form (rounded to the
float32 storage format, the same bytes on both sides); the compressor on its
outputs; the two together end to end against the oracle's float64 chain.
"""
import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import topk as otk
from tests.gpu_util import (KL_ABS, KL_REL, compare_topk_compress, compare_topk_grad, grad_to_f64, qrest_rel,
                            say, topk_kl_tol, topk_kl_tol_far_rest)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _upload(t: otk.TopK):
    return (torch.as_tensor(np.ascontiguousarray(t.idx, np.int32), device=DEV),
            torch.as_tensor(np.ascontiguousarray(t.logp, np.float32), device=DEV),
            torch.as_tensor(np.ascontiguousarray(t.rest, np.float32), device=DEV))


def _gpu_compress(b, k):
    with qqe.Evaluator(b.shape[1], max(b.shape[0], 1), b.dtype, b.dtype, device=DEV) as ev:
        idx, logp, rest = ev.topk_compress(b, k)
        torch.cuda.synchronize()
    return idx.cpu().numpy(), logp.cpu().numpy(), rest.cpu().numpy()


def _gpu_eval(stored, q, k, base_dtype):
    n = q.shape[0]
    kld = torch.empty(n, dtype=torch.float32, device=DEV)
    match = torch.empty(n, dtype=torch.uint8, device=DEV)
    ab = torch.empty(n, dtype=torch.int32, device=DEV)
    aq = torch.empty(n, dtype=torch.int32, device=DEV)
    with qqe.Evaluator(q.shape[1], max(n, 1), base_dtype, q.dtype, device=DEV) as ev:
        ev.rows_topk(*stored, q, 0, kld, match, ab, aq)
        summ = ev.reduce(n)
        torch.cuda.synchronize()
    return kld.cpu().numpy(), match.cpu().numpy(), ab.cpu().numpy(), aq.cpu().numpy(), summ


def _check_eval(g_kl, g_match, g_ab, g_aq, o_res, stored, nq, ctx, far_rest=False):
    """Coarsened KL per row against the oracle's on the same stored bytes: the
    plain per-token rule; with far_rest, the rule widened by the streamed rest
    mass's bound (topk_kl_tol_far_rest), reporting how many rows need it."""
    err = np.abs(g_kl.astype(np.float64) - o_res.kl)
    if far_rest:
        R = np.asarray(stored.rest, np.float64)
        tol, plain = topk_kl_tol_far_rest(o_res.kl, o_res.q_rest, R, qrest_rel(oracle.to_f64(nq), stored.idx))
        say(f"[topk] {ctx}: {int((err > plain).sum())} of {err.size} rows within the widened bound only")
    else:
        tol = topk_kl_tol(o_res.kl)
    bad = err > tol
    assert not bad.any(), (f"{ctx}: {int(bad.sum())} rows out of tolerance, e.g. row {np.nonzero(bad)[0][0]}: "
                           f"gpu {g_kl[bad][0]!r} oracle {o_res.kl[bad][0]!r} tol {tol[bad][0]!r}")
    assert np.array_equal(g_aq.astype(np.int64), o_res.argmax_quant), f"{ctx}: quant argmax differs"
    assert np.array_equal(g_match, o_res.match), f"{ctx}: match differs"
    assert np.array_equal(g_ab.astype(np.int64), np.asarray(stored.idx[:, 0], np.int64)), f"{ctx}: base argmax"
    return float((err / tol).max())


CASES = [("c1", 64, 32000, 128), ("c2", 24, 151936, 128), ("c3", 16, 151936, 128), ("c4", 16, 262144, 128),
         ("c5", 24, 151936, 128), ("c2", 20, 151928, 1000), ("c4", 20, 4104, 7)]


@pytest.mark.parametrize("name,n_rows,vocab,k", CASES)
def test_topk_compress_parity(name, n_rows, vocab, k):
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, _ = synth.generate(cfg, device=DEV)
    nb = synth.to_numpy_bits(b)
    lse = oracle.rows(nb, nb).lse_base
    o = otk.compress(nb, k, lse)
    compare_topk_compress(*_gpu_compress(b, k), o, lse, ctx=f"{name} k={k}")


@pytest.mark.parametrize("name,n_rows,vocab,k", CASES)
def test_topk_eval_parity_on_oracle_stored_rows(name, n_rows, vocab, k):
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    stored = otk.to_storage(otk.compress(nb, k, oracle.rows(nb, nb).lse_base))
    o = otk.kl_topk(stored, nq, oracle.rows(nq, nq).lse_base)
    g = _gpu_eval(_upload(stored), q, k, cfg.base_dtype)
    worst = _check_eval(*g[:4], o, stored, nq, ctx=f"{name} k={k}")
    s = g[4]
    assert s.n_match == int(o.match.sum())
    say(f"[topk] {name} k={k}: eval worst error/tolerance {worst:.3f}; mean KL_K {s.kld_mean:.6g}")


@pytest.mark.parametrize("name,n_rows,vocab,k", CASES[:5])
def test_topk_end_to_end(name, n_rows, vocab, k):
    """GPU compress + GPU evaluate vs the oracle's float64 chain. The stored
    log-probabilities differ by up to the compressor's bound, which moves KL_K
    by at most that bound times (1 + sum_k p_k |log p_k - log q_k|)."""
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    lse_b = oracle.rows(nb, nb).lse_base
    o_t = otk.compress(nb, k, lse_b)
    o = otk.kl_topk(o_t, nq, oracle.rows(nq, nq).lse_base)
    gi, gl, gr = _gpu_compress(b, k)
    stored = (torch.as_tensor(gi, device=DEV), torch.as_tensor(gl, device=DEV), torch.as_tensor(gr, device=DEV))
    g_kl = _gpu_eval(stored, q, k, cfg.base_dtype)[0].astype(np.float64)
    tol = (topk_kl_tol(o.kl)
           + _storage_shift_bound(o_t, nq, lse_b))
    err = np.abs(g_kl - o.kl)
    assert (err <= tol).all(), f"{name}: end to end, worst error/tolerance {(err / tol).max():.3f}"


def _storage_shift_bound(o_t, nq, lse_b):
    """First-order change of KL_K when the stored values move by the
    compressor's bounds: d KL_K / d log p_k = p_k (1 + log p_k - log q_k) and
    d KL_K / d R = 1 + log(R / Q_rest); log p moves by at most eps (the
    log-normaliser bound + float32 rounding), R by REST_REL relative."""
    from tests.gpu_util import REST_REL
    lse_q = oracle.rows(nq, nq).lse_base
    eps = 4 * 2.0 ** -23 * np.maximum(np.abs(lse_b), 1.0) + 1e-6 + 2.0 ** -23 * np.abs(o_t.logp).max(axis=1)
    out = np.empty(len(lse_b))
    zq = oracle.to_f64(nq)
    for r in range(len(lse_b)):
        logq = zq[r, o_t.idx[r]] - lse_q[r]
        p = np.exp(o_t.logp[r])
        other = np.ones(zq.shape[1], bool)
        other[o_t.idx[r]] = False
        Q = float(np.exp(zq[r, other] - lse_q[r]).sum())
        R = float(o_t.rest[r])
        rterm = abs(1.0 + np.log(R / Q)) * R * REST_REL if R > 0 and Q > 0 else 0.0
        out[r] = 2.0 * (eps[r] * float(np.sum(p * (1.0 + np.abs(o_t.logp[r] - logq)))) + rterm)
    return out


@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 8, 65, 513, 4104])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_topk_edge_vocab_sizes_and_ties(vocab, dtypes):
    g0 = np.random.default_rng(vocab + 5)
    n = 6
    zb = np.round(g0.normal(0, 2.0, (n, vocab)), 1)
    zb[1] = 0.0
    zb[1, ::3] = -0.0                         # signed zeros: equal values
    zb[2] = 1.5                               # constant row
    zq = zb + np.round(g0.normal(0, 0.3, (n, vocab)), 2)
    b = torch.tensor(zb, dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtypes[1]), device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    lse = oracle.rows(nb, nb).lse_base
    for k in sorted({1, min(vocab, 5), vocab if vocab <= 1024 else 1024}):
        o_t = otk.compress(nb, k, lse)
        compare_topk_compress(*_gpu_compress(b, k), o_t, lse, ctx=f"V={vocab} k={k} {dtypes}")
        stored = otk.to_storage(o_t)
        o = otk.kl_topk(stored, nq, oracle.rows(nq, nq).lse_base)
        g = _gpu_eval(_upload(stored), q, k, dtypes[0])
        _check_eval(*g[:4], o, stored, nq, ctx=f"V={vocab} k={k} {dtypes}")


@pytest.mark.parametrize("k", [1, 128, 256, 300])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_compress_row_orders(k, dtype):
    """Full-width rows whose order and ties drive the selection through every
    regime: random, ascending, descending, a rising trend under noise,
    constant and coarsely rounded (both overflow the per-wave candidate lists
    into the exact path); 600 copies of the maximum scattered over the row
    (more than 512 kept candidates: the bitonic sort) and 100 copies of the
    maximum with 400 ties at a lower value (up to 500 kept: two keys per
    thread in the rank sort); 600 maxima that all fall to one wave (its list
    overflows while the others' fit: the exact path); k = 300 takes the
    large-K form of the sampled bound (a denser sample, longer lists)."""
    v = 151936
    g0 = np.random.default_rng(k + 17)
    many_max = g0.normal(0, 1.0, v)
    many_max[g0.choice(v, 600, replace=False)] = 9.0
    two_levels = g0.normal(0, 1.0, v)
    at = g0.choice(v, 500, replace=False)
    two_levels[at[:100]] = 9.0
    two_levels[at[100:]] = 6.0
    one_wave = g0.normal(0, 1.0, v)            # 600 maxima, all in the first quarter of their 2048-element step
    first = np.nonzero(np.arange(v) % 2048 < 512)[0]
    one_wave[g0.choice(first, 600, replace=False)] = 9.0
    rows = [g0.normal(0, 3.0, v), np.arange(v) * 1e-3, -np.arange(v) * 1e-3,
            g0.normal(0, 1.0, v) + np.linspace(0.0, 6.0, v), np.full(v, 0.75),
            np.round(g0.normal(0, 1.0, v), 1), many_max, two_levels, one_wave]
    b = torch.tensor(np.stack(rows), dtype=synth.torch_dtype(dtype), device=DEV)
    nb = synth.to_numpy_bits(b)
    lse = oracle.rows(nb, nb).lse_base
    compare_topk_compress(*_gpu_compress(b, k), otk.compress(nb, k, lse), lse, ctx=f"row orders k={k} {dtype}")


FAR_V = 2048 * 9  # nine 2048-element steps: the sample reads steps 0, 4, 8 (0, 2, ..., 8 for k > 256)


def _far_rows(where, k, gaps, seed):
    """Base rows whose k largest logits lie gap nats above every other one, and
    quant rows near them. "sampled": the k lie in the steps the sample reads,
    one per thread, over noise of width 0.1 -- the sampled bound sits on the
    k-th and every other element is a far-below non-candidate. "exact": the k
    lie in steps the sample skips (k <= 256) over a plateau of zeros, so every
    element is a candidate, the lists overflow and the row takes the exact
    path with its threshold on the k-th."""
    g = np.random.default_rng(seed)
    zb = np.zeros((len(gaps), FAR_V))
    for r, gap in enumerate(gaps):
        if where == "sampled":
            zb[r] = g.normal(0, 0.1, FAR_V)
            pos = np.concatenate([8 * np.arange(256), 4096 + 8 * np.arange(256)])[:k]
        else:
            pos = 2048 + 8 * np.arange(k)
        zb[r, pos] = gap + g.uniform(0.0, 1.0, k)
    zq = zb + 0.05 * g.normal(size=zb.shape)
    return zb, zq


@pytest.mark.parametrize("where,k", [("sampled", 8), ("sampled", 300), ("exact", 8), ("exact", 300)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_rest_far_below_the_stored_tokens(where, k, dtype):
    """Rest masses 30, 60 and 89 nats below the stored tokens: fp32
    exponentials shifted by the row maximum would lose precision with the
    distance and flush to zero past 87.3 nats (a zero quantized rest mass
    turns KL_K infinite). The compressor, the evaluator and the top-K gradient
    against the oracle, the stored rest mass to its relative bound."""
    zb, zq = _far_rows(where, k, (89.0, 60.0, 30.0), seed=k)
    ctx = f"far rest {where} k={k} {dtype}"
    b = torch.tensor(zb, dtype=synth.torch_dtype(dtype), device=DEV)
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtype), device=DEV)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    lse_b = oracle.rows(nb, nb).lse_base
    o_t = otk.compress(nb, k, lse_b)
    assert (o_t.rest > 2.0 ** -126).all(), f"{ctx}: the rows should carry a normal float32 rest mass"
    gi, gl, gr = _gpu_compress(b, k)
    compare_topk_compress(gi, gl, gr, o_t, lse_b, ctx=ctx)
    stored = otk.TopK(gi, gl, gr)
    up = _upload(stored)
    lse_q = oracle.rows(nq, nq).lse_base
    o = otk.kl_topk(stored, nq, lse_q)
    _check_eval(*_gpu_eval(up, q, k, dtype)[:4], o, stored, nq, ctx=ctx, far_rest=True)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    with qqe.Evaluator(FAR_V, q.shape[0], dtype, dtype, device=DEV) as ev:
        ev.rows_topk(*up, q)
        ev.grad_topk(up[0], up[1], q, 0, 1.0, out, "f32")
        torch.cuda.synchronize()
    compare_topk_grad(grad_to_f64(out), stored, nq, lse_q, 1.0, "f32", ctx=ctx)
    say(f"[topk] {ctx}: rest {gr[0]:.3e} {gr[1]:.3e} {gr[2]:.3e} ok")


def test_topk_bad_stored_indices_poison_only_their_row():
    cfg = synth.CONFIGS["c4"].scaled(n_rows=4, vocab=4104)
    b, q = synth.generate(cfg, device=DEV)
    nb = synth.to_numpy_bits(b)
    stored = otk.to_storage(otk.compress(nb, 16, oracle.rows(nb, nb).lse_base))
    stored.idx[1, 3] = stored.idx[1, 5]       # repeated id
    stored.idx[2, 0] = 4104                   # out of range
    stored.idx[3, 7] = -1                     # negative
    kl, match = _gpu_eval(_upload(stored), q, 16, "bf16")[:2]
    assert np.isfinite(kl[0]) and np.all(np.isnan(kl[1:])) and np.all(match[1:] == 0)


def test_topk_argument_errors():
    lib = qqe.load_library()
    with qqe.Evaluator(64, 4, "f32", "f32", device=DEV) as ev:
        z = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
        i = torch.zeros((4, 8), dtype=torch.int32, device=DEV)
        f = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
        p = z.data_ptr()
        for k in (0, 65, 1025, -3):
            assert lib.kld_eval_topk_compress(ev.handle, p, 4, k, i.data_ptr(), f.data_ptr(), f.data_ptr(),
                                              None) == qqe.KLD_ERR_INVALID_ARG
            assert lib.kld_eval_rows_topk(ev.handle, i.data_ptr(), f.data_ptr(), f.data_ptr(), k, p, 4, 0, None, None,
                                          None, None, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_rows_topk(ev.handle, i.data_ptr(), f.data_ptr(), f.data_ptr(), 8, p, 4, 1, None, None,
                                      None, None, None) == qqe.KLD_ERR_RANGE
        assert lib.kld_eval_topk_compress(ev.handle, None, 4, 8, i.data_ptr(), f.data_ptr(), f.data_ptr(),
                                          None) == qqe.KLD_ERR_INVALID_ARG
    # a vocabulary whose token map cannot fit on chip is refused before any launch
    with qqe.Evaluator(1 << 23, 1, "bf16", "bf16", device=DEV) as ev:
        assert lib.kld_eval_rows_topk(ev.handle, 8, 8, 8, 8, 8, 1, 0, None, None, None, None,
                                      None) == qqe.KLD_ERR_INVALID_ARG


@pytest.mark.slow
def test_full_c2_topk_sampled_rows_and_properties():
    cfg = synth.CONFIGS["c2"]
    b, q = synth.generate(cfg, device=DEV)
    n, v, k = cfg.n_rows, cfg.vocab, 128
    with qqe.Evaluator(v, n, "bf16", "bf16", device=DEV) as ev:
        full_kl = torch.empty(n, dtype=torch.float32, device=DEV)
        full_m = torch.empty(n, dtype=torch.uint8, device=DEV)
        full_ab = torch.empty(n, dtype=torch.int32, device=DEV)
        ev.rows(b, q, 0, full_kl, full_m, full_ab)
        idx, logp, rest = ev.topk_compress(b, k)
        kk = torch.empty(n, dtype=torch.float32, device=DEV)
        km = torch.empty(n, dtype=torch.uint8, device=DEV)
        ev.rows_topk(idx, logp, rest, q, 0, kk, km)
        s = ev.reduce(n)
        torch.cuda.synchronize()
    full_kl, kk = full_kl.cpu().numpy().astype(np.float64), kk.cpu().numpy().astype(np.float64)
    # every row: same top-1 decision as the full path, the first stored token is
    # the full path's base argmax, and the coarsened KL never exceeds the full one
    assert np.array_equal(km.cpu().numpy(), full_m.cpu().numpy())
    assert np.array_equal(idx[:, 0].cpu().numpy(), full_ab.cpu().numpy())
    slack = np.maximum(KL_REL * full_kl, KL_ABS) + 1e-5
    assert np.all(kk <= full_kl + slack), f"KL_K above full KL in {(kk > full_kl + slack).sum()} rows"
    # sampled rows against the oracle: stored form and end-to-end value
    plan = synth.row_plan(cfg)
    rows = np.unique(np.concatenate([[0, n - 1], np.nonzero(plan.moved)[0][:6],
                                     np.random.default_rng(4).integers(0, n, 24)]))
    sel = torch.as_tensor(rows, device=DEV)
    nb = synth.to_numpy_bits(b.index_select(0, sel))
    nq = synth.to_numpy_bits(q.index_select(0, sel))
    lse_b = oracle.rows(nb, nb).lse_base
    o_t = otk.compress(nb, k, lse_b)
    compare_topk_compress(idx.index_select(0, sel).cpu().numpy(), logp.index_select(0, sel).cpu().numpy(),
                          rest.index_select(0, sel).cpu().numpy(), o_t, lse_b, ctx="c2 full, sampled rows")
    o = otk.kl_topk(o_t, nq, oracle.rows(nq, nq).lse_base)
    tol = (topk_kl_tol(o.kl)
           + _storage_shift_bound(o_t, nq, lse_b))
    err = np.abs(kk[rows] - o.kl)
    assert (err <= tol).all(), f"c2 full sampled rows: worst error/tolerance {(err / tol).max():.3f}"
    say(f"[topk] c2 full: mean KL_128 {s.kld_mean:.6g} vs full mean {full_kl.mean():.6g}; "
        f"{rows.size} sampled rows ok (worst error/tolerance {(err / tol).max():.3f})")
    del b, q
    torch.cuda.empty_cache()
