"""GPU parity of the token-conditioned metrics and the per-segment summaries.

The token values (log-probability of the actual next token under each model,
its probability change) are computed in the row kernel's epilogue from two
gathered logits and the float64 log-normalisers; they are compared with the
float64 oracle row by row, and the summaries with the oracle's under bounds
derived from the per-row ones. Segment summaries are compared with the oracle
per segment, with exact host arithmetic on the GPU's own per-token values, and
bit-for-bit with the whole-evaluation reductions.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import tokens as otok
from tests.gpu_util import (check_summary_against_oracle, check_token_summary, compare_rows, compare_token_rows,
                            run_gpu, say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _edge_tokens(n, v, seed):
    """Seeded ids with every state represented: -1, 0, V-1, V, V+7, uniform."""
    g = np.random.default_rng(seed)
    t = g.integers(0, v, n).astype(np.int64)
    special = [-1, 0, v - 1, v, v + 7, -(2 ** 31)]
    for i, val in enumerate(special[:n]):
        t[(i * 7919) % n] = val
    return t.astype(np.int32)


@pytest.mark.parametrize("name,n_rows,vocab", [
    ("c1", 64, 32000),
    ("c2", 48, 151936),
    ("c3", 32, 151936),
    ("c4", 40, 262144),
    ("c5", 40, 151936),
    ("c2", 70, 151928),
    ("c4", 20, 4104),
])
def test_token_parity_oracle_sized(name, n_rows, vocab):
    say(f"[tokens] {name} n={n_rows} V={vocab}")
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    t = synth.tokens(cfg)
    t[::9] = _edge_tokens(n_rows, vocab, 5)[::9]
    g = run_gpu(b, q, tokens=t)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    o = oracle.rows(nb, nq)
    compare_rows(g, o, ctx=name)
    tr, tb, tq, td = compare_token_rows(g, nb, nq, o, ctx=name)
    check_token_summary(g["token_summary"], tr, tb, tq, td, g, ctx=name)


def test_token_at_the_argmax_and_peak_rows():
    """c2 rows whose token is the planted peak: log p is close to 0 and, in a
    moved row, the quantized model loses almost all of that probability."""
    cfg = synth.CONFIGS["c2"].scaled(n_rows=256)
    plan = synth.row_plan(cfg)
    b, q = synth.generate(cfg, device=DEV)
    t = plan.peak[:256].astype(np.int32)
    g = run_gpu(b, q, tokens=t)
    moved = plan.moved[:256]
    assert moved.any()
    assert np.all(g["lpb"] > -1e-3)
    assert np.all(g["dp"][moved] < -0.99) and np.all(np.abs(g["dp"][~moved]) < 1e-2)
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    o = oracle.rows(nb, nq)
    tr, tb, tq, td = compare_token_rows(g, nb, nq, o, ctx="peak tokens")
    check_token_summary(g["token_summary"], tr, tb, tq, td, g, ctx="peak tokens")


@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 65, 513, 4096 + 8])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_token_edge_vocab_sizes_and_states(vocab, dtypes):
    g0 = np.random.default_rng(vocab)
    n = 37
    zb = torch.tensor(g0.normal(0, 3.0, (n, vocab)), dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    zq = (zb.float() + torch.tensor(g0.normal(0, 0.3, (n, vocab)), dtype=torch.float32, device=DEV)).to(
        synth.torch_dtype(dtypes[1]))
    t = _edge_tokens(n, vocab, vocab + 1)
    g = run_gpu(zb, zq, tokens=t)
    nb, nq = synth.to_numpy_bits(zb), synth.to_numpy_bits(zq)
    o = oracle.rows(nb, nq)
    tr, tb, tq, td = compare_token_rows(g, nb, nq, o, ctx=f"V={vocab} {dtypes}")
    check_token_summary(g["token_summary"], tr, tb, tq, td, g, ctx=f"V={vocab} {dtypes}")
    assert g["token_summary"].n_invalid == int(np.count_nonzero(t >= vocab))


def test_rows_without_tokens_are_not_scored_and_invalid_ids_raise():
    cfg = synth.CONFIGS["c4"].scaled(n_rows=16, vocab=4104)
    b, q = synth.generate(cfg, device=DEV)
    with qqe.Evaluator(cfg.vocab, 16, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b[:8], q[:8], 0)                                  # no tokens: not scored
        t = torch.tensor([0, 1, 2, cfg.vocab, -1, 5, 6, 7], dtype=torch.int32, device=DEV)
        ev.rows(b[8:], q[8:], 8, tokens=t)
        ts = ev.reduce_tokens(16, allow_invalid=True)
        assert ts.n_scored == 6 and ts.n_invalid == 1
        with pytest.raises(ValueError):
            ev.reduce_tokens(16)
        ev.rows(b[8:], q[8:], 8)                                  # rewritten without tokens
        ts = ev.reduce_tokens(16)
        assert ts.n_scored == 0 and ts.n_invalid == 0 and math.isnan(ts.ppl_quant)


def test_token_outputs_bit_identical_across_chunking_and_streams():
    cfg = synth.CONFIGS["c5"].scaled(n_rows=96, vocab=151936)
    b, q = synth.generate(cfg, device=DEV)
    t = torch.as_tensor(synth.tokens(cfg), device=DEV)
    res = []
    for chunks in ([96], [40, 56], [1, 31, 64]):
        lpb, lpq, dp = (torch.empty(96, dtype=torch.float32, device=DEV) for _ in range(3))
        streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        with qqe.Evaluator(cfg.vocab, 96, "bf16", "bf16", device=DEV) as ev:
            r0 = 0
            for i, c in enumerate(chunks):
                s = streams[i % 2]
                sl = slice(r0, r0 + c)
                with torch.cuda.stream(s):
                    ev.rows(b[sl], q[sl], r0, stream=s, tokens=t[sl], logp_base_out=lpb[sl], logp_quant_out=lpq[sl],
                            dp_out=dp[sl])
                r0 += c
            ts = ev.reduce_tokens(96)
            torch.cuda.synchronize()
        res.append((lpb.cpu().numpy().tobytes(), lpq.cpu().numpy().tobytes(), dp.cpu().numpy().tobytes(),
                    (ts.logp_base_sum, ts.logp_quant_sum, ts.dp_mean, ts.dp_rms)))
    assert res[0] == res[1] == res[2]


# ---------------------------------------------------------------- segments ---

def _segment_case(n=3000, vocab=4104):
    cfg = synth.CONFIGS["c4"].scaled(n_rows=n, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    t = synth.tokens(cfg)
    t[::97] = -1
    return cfg, b, q, t


def test_segment_summaries_match_oracle_per_segment():
    cfg, b, q, t = _segment_case()
    n = cfg.n_rows
    offs = [0, 512, 1024, 1024, 1500, 2048 + 3, 2999, 3000]     # includes an empty and a one-row segment
    tok = torch.as_tensor(t, device=DEV)
    kld = torch.empty(n, dtype=torch.float32, device=DEV)
    match = torch.empty(n, dtype=torch.uint8, device=DEV)
    lpb, lpq, dp = (torch.empty(n, dtype=torch.float32, device=DEV) for _ in range(3))
    with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0, kld, match, tokens=tok, logp_base_out=lpb, logp_quant_out=lpq, dp_out=dp)
        segs = ev.reduce_segments(offs)
        whole_k, whole_t = ev.reduce(n), ev.reduce_tokens(n)
        one = ev.reduce_segments([0, n])
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    o = oracle.rows(nb, nq)
    g = dict(kld=kld.cpu().numpy(), match=match.cpu().numpy(), lpb=lpb.cpu().numpy(), lpq=lpq.cpu().numpy(),
             dp=dp.cpu().numpy(), tokens=t)
    tr, tb, tq, td = compare_token_rows(g, nb, nq, o, ctx="segments")
    # one segment over every row is the whole-evaluation reduction, bit for bit
    assert one[0][0] == whole_k and one[0][1] == whole_t
    for k, (ks, ts) in enumerate(segs):
        a, z = offs[k], offs[k + 1]
        ctx = f"segment {k} [{a}, {z})"
        assert ks.n_rows == z - a
        if z == a:
            assert math.isnan(ks.kld_mean) and ks.kld_max_row == -1 and ks.n_match == 0 and ts.n_scored == 0
            assert ks.kld_max == -math.inf and math.isnan(ks.same_top1)
            continue
        sub = oracle.RowResults(o.kl[a:z], None, None, o.match[a:z], None, None)
        check_summary_against_oracle(ks, sub, ctx=ctx, strict_mean=False, row_base=a)
        gk = g["kld"][a:z].astype(np.float64)
        exact = math.fsum(gk.tolist())
        assert abs(ks.kld_sum - exact) <= 1e-12 * abs(exact) + 1e-300, ctx
        assert ks.kld_max == gk.max() and ks.kld_max_row == a + int(np.argmax(gk)), ctx
        assert ks.n_match == int(g["match"][a:z].astype(np.int64).sum()), ctx
        trs = otok.TokenRows(tr.logp_base[a:z], tr.logp_quant[a:z], tr.dp[a:z], tr.state[a:z])
        gs = {key: g[key][a:z] for key in ("lpb", "lpq", "dp")}
        check_token_summary(ts, trs, tb[a:z], tq[a:z], td[a:z], gs, ctx=ctx)


def test_segment_summaries_are_chunking_invariant_and_workspace_regrows():
    cfg, b, q, t = _segment_case(2200, 1000)
    n = cfg.n_rows
    tok = torch.as_tensor(t, device=DEV)
    many = list(range(0, n + 1, 3)) + ([n] if n % 3 else [])    # 734 short segments
    out = []
    for chunks in ([n], [700, 1500], [1, 1024, 1175]):
        with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
            r0 = 0
            for c in chunks:
                ev.rows(b[r0:r0 + c], q[r0:r0 + c], r0, tokens=tok[r0:r0 + c])
                r0 += c
            a = ev.reduce_segments([0, 1000, n])
            m = ev.reduce_segments(many)                       # grows the workspace
            a2 = ev.reduce_segments([0, 1000, n])              # reuses it
            assert a == a2
            w = ev.reduce(n)
        assert len(m) == len(many) - 1
        assert sum(k.n_rows for k, _ in m) == n and sum(k.n_match for k, _ in m) == w.n_match
        out.append((a, m))
    assert out[0] == out[1] == out[2]


def test_repeated_reductions_reuse_tables_and_see_new_rows():
    """A reduction over the offsets of the previous one reuses its uploaded
    tile tables: the results must equal a fresh computation, and rows written
    into the handle in between must show."""
    cfg, b, q, _ = _segment_case(2200, 1000)
    n = cfg.n_rows
    with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0)
        w1, p1 = ev.reduce(n), ev.reduce(1500)
        assert ev.reduce(n) == w1 and ev.reduce(n) == w1
        segs = ev.reduce_segments([0, 1500, n])
        assert segs[0][0] == p1 and ev.reduce(1500) == p1
        ev.rows(q, b, 0)                                   # new values, same offsets
        w2 = ev.reduce(n)
        assert w2 != w1
        with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as fresh:
            fresh.rows(q, b, 0)
            assert fresh.reduce(n) == w2 and fresh.reduce(1500) == ev.reduce(1500)


def test_reductions_reuse_results_until_rows_are_written():
    """A reduction over the rows of the previous one, with no row written in
    between, returns that one's results; any rows or rows_topk call makes the
    next reduction compute afresh."""
    cfg, b, q, t = _segment_case(2200, 1000)
    n = cfg.n_rows
    tok = torch.as_tensor(t, device=DEV)
    with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0, tokens=tok)
        k1, t1 = ev.reduce(n), ev.reduce_tokens(n)
        assert ev.reduce_segments([0, n])[0] == (k1, t1)
        with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as fresh:
            fresh.rows(b, q, 0, tokens=tok)
            assert fresh.reduce_tokens(n) == t1 and fresh.reduce(n) == k1
        ev.rows(b[:100], q[:100], 0)                       # rows 0..99 again, now without next-token ids
        t2 = ev.reduce_tokens(n)
        assert t2.n_scored == t1.n_scored - int(((t[:100] >= 0) & (t[:100] < cfg.vocab)).sum())
        idx, logp, rest = ev.topk_compress(b[:50], 4)
        k3 = ev.reduce(n)
        assert k3 == k1                                    # the same per-token KLD values as at first
        ev.rows_topk(idx, logp, rest, q[:50], 0)
        k4 = ev.reduce(n)
        assert k4 != k3 and k4.n_rows == n


def test_segment_argument_errors():
    with qqe.Evaluator(64, 10, "f32", "f32", device=DEV) as ev:
        z = torch.zeros((10, 64), dtype=torch.float32, device=DEV)
        ev.rows(z, z, 0)
        lib = qqe.load_library()
        import ctypes
        for offs, st in (([0, 5, 3], qqe.KLD_ERR_INVALID_ARG), ([0, 11], qqe.KLD_ERR_RANGE),
                         ([-1, 4], qqe.KLD_ERR_RANGE)):
            arr = (ctypes.c_int64 * len(offs))(*offs)
            assert lib.kld_eval_reduce_segments(ev.handle, arr, len(offs) - 1, None, None, None) == st
        arr = (ctypes.c_int64 * 2)(0, 4)
        assert lib.kld_eval_reduce_segments(ev.handle, arr, 0, None, None, None) == qqe.KLD_ERR_INVALID_ARG
        assert lib.kld_eval_reduce_segments(ev.handle, None, 1, None, None, None) == qqe.KLD_ERR_INVALID_ARG
        segs = ev.reduce_segments([0, 10])
        assert segs[0][0].n_rows == 10 and segs[0][0].kld_sum == 0.0 and segs[0][0].n_match == 10


def test_concurrent_host_threads_on_one_handle():
    """Several host threads feed disjoint row ranges of one handle on their own
    streams and reduce concurrently; results equal a single-threaded run bit
    for bit (ctypes releases the GIL during the library calls)."""
    import threading
    cfg = synth.CONFIGS["c5"].scaled(n_rows=256, vocab=151936)
    b, q = synth.generate(cfg, device=DEV)
    t = torch.as_tensor(synth.tokens(cfg), device=DEV)
    n = cfg.n_rows
    with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 0, tokens=t)
        ref = (ev.reduce(n), ev.reduce_tokens(n), ev.reduce_segments([0, 100, n]))
    with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
        errors = []
        pieces = [(0, 40), (40, 101), (101, 200), (200, 256)]
        start = threading.Barrier(len(pieces))

        def feed(a, z):
            try:
                torch.cuda.set_device(DEV)
                s = torch.cuda.Stream(device=DEV)
                s.wait_stream(torch.cuda.default_stream(DEV))
                start.wait()
                with torch.cuda.stream(s):
                    ev.rows(b[a:z], q[a:z], a, stream=s, tokens=t[a:z])
            except Exception as e:  # surfaced below
                errors.append(e)

        torch.cuda.synchronize()
        th = [threading.Thread(target=feed, args=p) for p in pieces]
        for x in th:
            x.start()
        for x in th:
            x.join()
        assert not errors, errors
        got = []

        def red():
            try:
                got.append((ev.reduce(n), ev.reduce_tokens(n), ev.reduce_segments([0, 100, n])))
            except Exception as e:
                errors.append(e)

        rt = [threading.Thread(target=red) for _ in range(3)]
        for x in rt:
            x.start()
        for x in rt:
            x.join()
        assert not errors, errors
    assert len(got) == 3 and all(g == ref for g in got)
