"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle on
host copies of the same bytes, compare to the stated tolerances."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import tokens as otok

# Per-token KLD: |gpu - oracle| <= 1e-5 |oracle| or <= 1e-7; mean KLD within
# 1e-6 relative; argmax, match flags and match counts bit-exact.
KL_REL, KL_ABS, MEAN_REL = 1e-5, 1e-7, 1e-6
# log-normalisers: float32 results of O(10..300) values; 4 ulp of the value
LSE_REL = 4 * 2.0 ** -23


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def kl_ok(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = np.abs(g - o)
    return (err <= KL_REL * np.abs(o)) | (err <= KL_ABS)


def assert_kl_close(g, o, ctx=""):
    ok = kl_ok(g, o)
    if not ok.all():
        bad = np.nonzero(~ok)[0][:8]
        raise AssertionError(f"{ctx}: {int((~ok).sum())} rows out of tolerance, e.g. rows {bad.tolist()} "
                             f"gpu={np.asarray(g)[bad].tolist()} oracle={np.asarray(o)[bad].tolist()}")


def error_stats(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = np.abs(g - o)
    rel = err / np.maximum(np.abs(o), 1e-300)
    return float(err.max()), float(np.where(err > KL_ABS, rel, 0).max())


def run_gpu(base: torch.Tensor, quant: torch.Tensor, row_offset=0, ev=None, stream=None, tokens=None):
    """Per-token results of the HIP path for all rows of base/quant. With
    ``tokens`` (host int array) the token-conditioned outputs and, for an
    evaluator owned here, the token summary are returned too."""
    n = base.shape[0]
    dev = base.device
    kld = torch.empty(n, dtype=torch.float32, device=dev)
    match = torch.empty(n, dtype=torch.uint8, device=dev)
    ab = torch.empty(n, dtype=torch.int32, device=dev)
    aq = torch.empty(n, dtype=torch.int32, device=dev)
    tok = None if tokens is None else torch.as_tensor(np.asarray(tokens, np.int32), device=dev)
    lpb = lpq = dp = None
    if tok is not None:
        lpb, lpq, dp = (torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3))
    own = ev is None
    if own:
        ev = qqe.Evaluator(base.shape[1], max(n + row_offset, 1), base.dtype, quant.dtype, device=dev)
    ev.rows(base, quant, row_offset, kld, match, ab, aq, stream=stream, tokens=tok, logp_base_out=lpb,
            logp_quant_out=lpq, dp_out=dp)
    summ = ev.reduce(n + row_offset) if own and n > 0 else None
    tsum = ev.reduce_tokens(n + row_offset, allow_invalid=True) if own and n > 0 and tok is not None else None
    lse_b = torch.empty(n, dtype=torch.float32, device=dev)
    lse_q = torch.empty(n, dtype=torch.float32, device=dev)
    ev.copy_lse(row_offset, n, lse_b, lse_q)
    flags = ev.row_flags(row_offset, n)
    torch.cuda.synchronize()
    res = dict(kld=kld.cpu().numpy(), match=match.cpu().numpy(), ab=ab.cpu().numpy(), aq=aq.cpu().numpy(),
               lse_b=lse_b.cpu().numpy(), lse_q=lse_q.cpu().numpy(), summary=summ, flags=flags.cpu().numpy())
    if tok is not None:
        res.update(lpb=lpb.cpu().numpy(), lpq=lpq.cpu().numpy(), dp=dp.cpu().numpy(), tokens=np.asarray(tokens),
                   token_summary=tsum)
    if own:
        ev.close()
    return res


def oracle_rows(base: torch.Tensor, quant: torch.Tensor, rows=None):
    if rows is not None:
        idx = torch.as_tensor(np.asarray(rows), device=base.device)
        base = base.index_select(0, idx)
        quant = quant.index_select(0, idx)
    return oracle.rows(synth.to_numpy_bits(base), synth.to_numpy_bits(quant))


def compare_rows(g, o, rows=None, ctx=""):
    """Element-by-element comparison of GPU per-token results with the oracle's."""
    sel = slice(None) if rows is None else np.asarray(rows)
    gk, gm = g["kld"][sel], g["match"][sel]
    gb, gq = g["ab"][sel], g["aq"][sel]
    assert np.array_equal(gb.astype(np.int64), o.argmax_base), f"{ctx}: base argmax differs"
    assert np.array_equal(gq.astype(np.int64), o.argmax_quant), f"{ctx}: quant argmax differs"
    assert np.array_equal(gm, o.match), f"{ctx}: match flags differ"
    assert_kl_close(gk, o.kl, ctx)
    for name, gl, ol in (("lse_base", g["lse_b"][sel], o.lse_base), ("lse_quant", g["lse_q"][sel], o.lse_quant)):
        err = np.abs(gl.astype(np.float64) - ol)
        tol = LSE_REL * np.maximum(np.abs(ol), 1.0) + 1e-6
        assert (err <= tol).all(), f"{ctx}: {name} max err {err.max()}"
    return error_stats(gk, o.kl)


def check_summary_against_oracle(summ, o, ctx="", strict_mean=True, row_base=0):
    """Summary vs the oracle's. The 1e-6 relative bound on the mean is the one
    stated for the five workloads and is asserted on them at full size; on a
    scaled-down sample (strict_mean=False) the mean is implied by the per-token
    check and its relative error is only reported."""
    s = oracle.summary(o.kl, o.match)
    assert summ.n_rows == s.n_rows
    assert summ.n_match == s.n_match, f"{ctx}: n_match {summ.n_match} vs {s.n_match}"
    assert summ.same_top1 == s.same_top1
    mean_rel = abs(summ.kld_mean - s.kld_mean) / max(abs(s.kld_mean), 1e-300)
    say(f"[summary] {ctx}: mean {summ.kld_mean:.10g} vs oracle {s.kld_mean:.10g} (rel err {mean_rel:.2e})")
    if strict_mean:
        assert mean_rel <= MEAN_REL, f"{ctx}: mean {summ.kld_mean!r} vs {s.kld_mean!r}"
    assert kl_ok([summ.kld_max], [s.kld_max]).all(), f"{ctx}: max {summ.kld_max} vs {s.kld_max}"
    top2 = np.sort(o.kl)[-2:] if o.kl.size > 1 else o.kl
    if o.kl.size == 1 or not kl_ok([top2[0]], [top2[1]]).all():
        assert summ.kld_max_row == row_base + s.kld_max_row, \
            f"{ctx}: max row {summ.kld_max_row} vs {row_base} + {s.kld_max_row}"


def check_summary_properties(summ, g, ctx=""):
    """Summary of the reduce kernel vs exact host arithmetic on the GPU's own per-token values."""
    k = g["kld"].astype(np.float64)
    n = k.size
    assert summ.n_rows == n
    assert summ.n_match == int(g["match"].astype(np.int64).sum())
    exact = math.fsum(k.tolist())
    assert abs(summ.kld_sum - exact) <= 1e-12 * max(abs(exact), 1e-300) + 1e-300, f"{ctx}: sum"
    assert summ.kld_max == k.max()
    assert summ.kld_max_row == int(np.argmax(k))
    assert summ.same_top1 == summ.n_match / n


# ---------------------------------------------------------------- tokens ---
# log p(t) = z[t] - lse is formed on the GPU from the float64 log-normaliser,
# so its error is the log-normaliser's (bounded above, LSE_REL of the value +
# 1e-6) plus one float32 rounding of log p(t). dp = q(t) - p(t) then errs by
# at most p * err(log p) + q * err(log q) (to first order) plus one float32
# rounding. Summary bounds follow from the per-row ones: a sum errs by at most
# the sum of its terms' bounds, an RMS by at most the RMS of the dp bounds
# (triangle inequality in L2).


def logp_tol(lp_o, lse_o):
    return LSE_REL * np.maximum(np.abs(lse_o), 1.0) + 1e-6 + 2.0 ** -24 * np.abs(lp_o)


def compare_token_rows(g, nb, nq, o, rows=None, ctx=""):
    """GPU token outputs vs the oracle's for the host rows nb/nq (bits or
    floats) whose oracle results are ``o``. Returns (oracle TokenRows, tol_b,
    tol_q, tol_dp) for the summary check."""
    sel = slice(None) if rows is None else np.asarray(rows)
    t = g["tokens"][sel]
    tr = otok.token_rows(nb, nq, t, o.lse_base, o.lse_quant)
    gb, gq, gd = (g[k][sel].astype(np.float64) for k in ("lpb", "lpq", "dp"))
    scored = tr.state == otok.SCORED
    for name, a in (("logp_base", gb), ("logp_quant", gq), ("dp", gd)):
        assert np.array_equal(np.isnan(a), ~scored), f"{ctx}: {name} NaN pattern differs from the scored rows"
    tb = np.where(scored, logp_tol(tr.logp_base, o.lse_base), 0.0)
    tq = np.where(scored, logp_tol(tr.logp_quant, o.lse_quant), 0.0)
    pb = np.where(scored, np.exp(tr.logp_base), 0.0)
    pq = np.where(scored, np.exp(tr.logp_quant), 0.0)
    td = np.where(scored, pb * tb + pq * tq + 2.0 ** -24 * np.abs(np.nan_to_num(tr.dp)) + 1e-30, 0.0)
    for name, a, ref, tol in (("logp_base", gb, tr.logp_base, tb), ("logp_quant", gq, tr.logp_quant, tq),
                              ("dp", gd, tr.dp, td)):
        err = np.abs(a[scored] - ref[scored])
        bad = err > tol[scored]
        if bad.any():
            i = np.nonzero(scored)[0][np.nonzero(bad)[0][:6]]
            raise AssertionError(f"{ctx}: {name} out of tolerance in {int(bad.sum())} rows, e.g. rows {i.tolist()} "
                                 f"gpu={a[i].tolist()} oracle={ref[i].tolist()} tol={tol[i].tolist()}")
    return tr, tb, tq, td


def _log_clamped(x):
    """log x clamped to [log of the smallest subnormal, log of the largest double]."""
    if x == math.inf:
        return math.log(sys.float_info.max)
    if x <= 0.0:
        return math.log(5e-324)
    return min(max(math.log(x), math.log(5e-324)), math.log(sys.float_info.max))


def check_token_summary(ts, tr, tb, tq, td, g=None, ctx=""):
    """Token summary vs the oracle's (bounds derived from the per-row ones) and,
    given the GPU's own per-token values, vs exact host arithmetic on them."""
    s = otok.token_summary(tr)
    assert ts.n_scored == s.n_scored, f"{ctx}: n_scored {ts.n_scored} vs {s.n_scored}"
    assert ts.n_invalid == s.n_invalid, f"{ctx}: n_invalid {ts.n_invalid} vs {s.n_invalid}"
    n = s.n_scored
    if n == 0:
        assert math.isnan(ts.ppl_base) and math.isnan(ts.dp_rms)
        return
    slack = 1e-12
    eb, eq = float(tb.sum()), float(tq.sum())
    assert abs(ts.logp_base_sum - s.logp_base_sum) <= eb + slack * abs(s.logp_base_sum), f"{ctx}: logp_base_sum"
    assert abs(ts.logp_quant_sum - s.logp_quant_sum) <= eq + slack * abs(s.logp_quant_sum), f"{ctx}: logp_quant_sum"
    # in log space, clamped to the double range: a perplexity may overflow to +inf
    # (or a ratio underflow to 0) on one side only, within the tolerance
    assert abs(_log_clamped(ts.ppl_base) - _log_clamped(s.ppl_base)) <= eb / n + slack, \
        f"{ctx}: ppl_base {ts.ppl_base} vs {s.ppl_base}"
    assert abs(_log_clamped(ts.ppl_quant) - _log_clamped(s.ppl_quant)) <= eq / n + slack, f"{ctx}: ppl_quant"
    assert abs(_log_clamped(ts.ppl_ratio) - _log_clamped(s.ppl_ratio)) <= (eb + eq) / n + slack, f"{ctx}: ppl_ratio"
    assert abs(ts.dp_mean - s.dp_mean) <= float(td.sum()) / n + 1e-15, f"{ctx}: dp_mean {ts.dp_mean} vs {s.dp_mean}"
    assert abs(ts.dp_rms - s.dp_rms) <= math.sqrt(float((td * td).sum()) / n) + 1e-15, f"{ctx}: dp_rms"
    say(f"[tokens] {ctx}: n_scored {n} PPL(Q) {ts.ppl_quant:.8g} (oracle {s.ppl_quant:.8g}) ratio {ts.ppl_ratio:.8g} "
        f"dp mean {ts.dp_mean:.4e} rms {ts.dp_rms:.4e}")
    if g is not None:
        sc = ~np.isnan(g["lpb"])
        for got, vals in ((ts.logp_base_sum, g["lpb"][sc]), (ts.logp_quant_sum, g["lpq"][sc])):
            ex = math.fsum(vals.astype(np.float64).tolist())
            assert abs(got - ex) <= 1e-12 * max(abs(ex), 1e-300), f"{ctx}: reduction of the GPU's own values"
        d = g["dp"][sc].astype(np.float64)
        # float64 sums of mixed-sign terms: error bounded relative to the sum of magnitudes
        assert abs(ts.dp_mean - math.fsum(d.tolist()) / n) <= 1e-12 * float(np.abs(d).sum()) / n + 1e-300
        assert abs(ts.dp_rms - math.sqrt(math.fsum((d * d).tolist()) / n)) <= 1e-12 * ts.dp_rms + 1e-300


# --------------------------------------------------------------- gradient ---
# g = scale (q - p) with p = 2^((zb - lse_b) log2 e) in fp32: each probability
# carries the log-normaliser's error (LSE bound above) plus the rounding of its
# exponent argument (<= 2^-23 (|z - lse| + 1) relative), the difference and
# the scaling add 2^-23 |g|, a bfloat16 output adds its half-ulp 2^-8 |g|, and
# values near the float32 underflow threshold may flush to zero.


def grad_tol(zb, zq, lse_b, lse_q, p, q, ref, scale, out_dtype):
    lb = np.asarray(lse_b, np.float64)[:, None]
    lq = np.asarray(lse_q, np.float64)[:, None]
    eb = LSE_REL * np.maximum(np.abs(lb), 1.0) + 1e-6 + 2.0 ** -23 * (np.abs(zb - lb) + 1.0)
    eq = LSE_REL * np.maximum(np.abs(lq), 1.0) + 1e-6 + 2.0 ** -23 * (np.abs(zq - lq) + 1.0)
    rnd = 2.0 ** -23 + (2.0 ** -8 if out_dtype == "bf16" else 0.0)
    return abs(scale) * (p * eb + q * eq) + rnd * np.abs(ref) + 2.0 ** -125 * max(abs(scale), 1.0)


def grad_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare_grad(g, nb, nq, o, scale, out_dtype, ctx=""):
    """GPU gradient rows (float64 host array) vs the oracle's for host rows nb/nq
    with oracle row results ``o``. Returns the largest error / tolerance ratio."""
    from oracle import grad as ograd
    ref, p, q = ograd.grad_rows(nb, nq, o.lse_base, o.lse_quant, scale)
    tol = grad_tol(oracle.to_f64(nb), oracle.to_f64(nq), o.lse_base, o.lse_quant, p, q, ref, scale, out_dtype)
    err = np.abs(g - ref)
    bad = err > tol
    if bad.any():
        r, i = np.nonzero(bad)
        raise AssertionError(f"{ctx}: {int(bad.sum())} gradient entries out of tolerance, e.g. row {r[0]} "
                             f"index {i[0]}: gpu {g[r[0], i[0]]!r} oracle {ref[r[0], i[0]]!r} "
                             f"tol {tol[r[0], i[0]]!r}")
    return float((err / tol).max())


# ------------------------------------------------------------------ top-K ---
# Compressor: indices are decided by exact comparisons of the inputs (bit-exact);
# Streamed masses are float64 sums of 8-term fp32 sums of exponentials
# exp(z - s), each relative to a shift s at or above its term. Per term the
# relative error is below EXP_ARG_REL per nat of s - z (the fp32 argument
# (z - s) log2(e) is rounded relative to its size: two roundings of 2^-24 and
# the 1.3e-8 error of log2(e) in float32) plus EXP_SUM_REL (one ulp of the
# exponential, 2^-23, and the 8-term sum, 7 x 2^-24). For N terms of sum W
# (relative to s) the mass-weighted mean distance is at most ln(N / W) -- the
# most when all terms are equal -- and terms more than 87.3 nats below s
# flush to zero.
EXP_ARG_REL = 1.33e-7
EXP_SUM_REL = 5.4e-7
# log p = z - lse carries the log-normaliser's error (LSE bound) plus one float32
# rounding. The rest mass R is a ratio whose numerator is the only fp32-streamed
# sum: its terms are shifted by the K-th largest value (or the sampled bound just
# below it, which lies above every term), and a sum with W < N e^-20 is taken
# again relative to its own maximum (W >= 1 there, N < 2^31): relative error at
# most EXP_ARG_REL x 21.5 + EXP_SUM_REL = 3.4e-6 in every row; 4e-6, plus its
# float32 rounding (the float64 ratio keeps its accuracy into float32's
# subnormal range, where the rounding is absolute: 2^-149).
REST_REL = 4e-6
# Evaluator (same stored bytes on both sides): the stored tokens are evaluated
# in float64; only the streamed mass Q_rest outside them carries fp32 rounding,
# and it enters KL_K with the coefficient (Q_rest - R): error <= qrest_rel
# |Q_rest - R| on top of the per-token rule of the main path. Its terms are
# shifted by running maxima at most the row maximum, so the bound is per row
# (qrest_rel); a sum under (V - K) e^-60, where terms could flush, is taken
# again relative to its own maximum, which only lowers the distances.


def compare_topk_compress(idx, logp, rest, o_topk, lse_base, ctx=""):
    """GPU stored form (host arrays) vs the oracle's float64 one."""
    assert np.array_equal(idx.astype(np.int64), o_topk.idx), f"{ctx}: stored indices differ"
    tol = LSE_REL * np.maximum(np.abs(lse_base), 1.0)[:, None] + 1e-6 + 2.0 ** -23 * np.abs(o_topk.logp)
    err = np.abs(logp.astype(np.float64) - o_topk.logp)
    assert (err <= tol).all(), f"{ctx}: logp max err {err.max():.3e} (worst ratio {(err / tol).max():.3f})"
    rel = np.abs(rest.astype(np.float64) - o_topk.rest)
    rtol = (REST_REL + 2.0 ** -23) * o_topk.rest + 2.0 ** -149
    assert (rel <= rtol).all(), f"{ctx}: rest max rel err {np.max(rel / np.maximum(o_topk.rest, 1e-300)):.3e}"


def qrest_rel(zq, idx):
    """Per-row relative error bound of the evaluator's Q_rest for quant rows zq
    (float64, n x V; host arrays) and stored token ids idx (n x K):
    EXP_ARG_REL times the mass-weighted mean of M - z over the tokens outside
    the stored ones (M the row maximum), plus EXP_SUM_REL."""
    zq = np.asarray(zq, np.float64)
    M = zq.max(axis=1, keepdims=True)
    w = np.exp(zq - M)
    np.put_along_axis(w, np.asarray(idx, np.int64), 0.0, axis=1)
    wd = np.where(w > 0, w * (M - zq), 0.0)
    W = w.sum(axis=1)
    return EXP_ARG_REL * np.where(W > 0, wd.sum(axis=1) / np.where(W > 0, W, 1.0), 0.0) + EXP_SUM_REL


def qrest_rel_device(q, idx, chunk=256):
    """qrest_rel for device rows q (n x V, any float dtype) and device ids idx,
    with torch in float64, a chunk of rows at a time."""
    import torch
    out = []
    for r0 in range(0, q.shape[0], chunk):
        z = q[r0:r0 + chunk].double()
        M = z.max(dim=1, keepdim=True).values
        w = torch.exp(z - M)
        w.scatter_(1, idx[r0:r0 + chunk].long(), 0.0)
        wd = torch.where(w > 0, w * (M - z), torch.zeros_like(w))
        W = w.sum(dim=1)
        D = torch.where(W > 0, wd.sum(dim=1) / torch.where(W > 0, W, torch.ones_like(W)), torch.zeros_like(W))
        out.append(D.cpu().numpy())
        del z, w, wd
    return EXP_ARG_REL * np.concatenate(out) + EXP_SUM_REL


def topk_kl_tol(o_kl):
    """The per-token rule of the full divergence, unchanged: the coarsened KL is
    a KL divergence (of two distributions over the stored tokens plus one
    outcome), held to the same 1e-5 relative / 1e-7 absolute bound."""
    return np.maximum(KL_REL * np.abs(o_kl), KL_ABS)


def topk_kl_tol_far_rest(o_kl, q_rest, R, qrel):
    """The per-token rule widened by qrel |Q_rest - R| (qrel: per-row bound of
    Q_rest's relative error, qrest_rel). Used only for rows whose rest of the
    mass lies tens of nats below the stored tokens: there each fp32 term of the
    streamed Q_rest carries 1.33e-7 per nat of that distance (the float32
    argument's rounding), which exceeds 1e-5 |KL_K| at 60-90 nats, while the
    stored tokens are evaluated in float64. Returns (tolerance, plain rule)."""
    plain = topk_kl_tol(o_kl)
    return plain + qrel * np.abs(q_rest - R), plain


# ----------------------------------------------------------- top-K gradient ---
# Stored token j: g = scale (q_j (P + R) - p_j); q_j is an fp32 exponential
# with the quant row's log-space error eq (as in the dense gradient), p_j and
# P, R are the stored values widened exactly, the rest is float64.
# Other token i: g = scale q_i F with F = P + R - R / Q_rest rounded to
# float32; Q_rest comes from the evaluator's fp32-streamed sum (relative error
# at most qrest_rel of the row), which moves F by up to (R / Q_rest) qrest_rel.
# Output rounding as for the dense gradient; an fp32 probability under 2^-126
# may flush to zero, which the dense gradient's floor covers for factors up to
# 1 but F can be far larger (R >> Q_rest): |F| 2^-126 more per entry.


def topk_grad_tol(stored, nq, lse_q, ref, scale, out_dtype):
    zq = oracle.to_f64(nq)
    lq = np.asarray(lse_q, np.float64)[:, None]
    q = np.exp(zq - lq)
    eq = LSE_REL * np.maximum(np.abs(lq), 1.0) + 1e-6 + 2.0 ** -23 * (np.abs(zq - lq) + 1.0)
    n, v = zq.shape
    tol = np.empty((n, v))
    qrel = qrest_rel(zq, stored.idx)
    for r in range(n):
        sel = np.asarray(stored.idx[r], np.int64)
        P = float(np.exp(np.asarray(stored.logp[r], np.float64)).sum())
        R = float(stored.rest[r])
        other = np.ones(v, bool)
        other[sel] = False
        Q = float(q[r, other].sum())
        F = P + R - (R / Q if R > 0 else 0.0)
        tol[r] = q[r] * (abs(F) * (eq[r] + 2.0 ** -23) + (R / Q if R > 0 else 0.0) * qrel[r]) + abs(F) * 2.0 ** -126
        tol[r, sel] = q[r, sel] * (P + R) * eq[r, sel]
    rnd = 2.0 ** -23 + (2.0 ** -8 if out_dtype == "bf16" else 0.0)
    return abs(scale) * tol + rnd * np.abs(ref) + 2.0 ** -125 * max(abs(scale), 1.0)


def compare_topk_grad(g, stored, nq, lse_q, scale, out_dtype, ctx=""):
    """GPU top-K gradient rows (float64 host array) vs the oracle's for the
    stored rows ``stored`` and host quant rows ``nq``; returns the largest
    error / tolerance ratio."""
    from oracle import topk as otk
    ref = otk.grad_topk(stored, nq, lse_q, scale)
    tol = topk_grad_tol(stored, nq, lse_q, ref, scale, out_dtype)
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    if bad.any():
        r, i = np.nonzero(bad)
        raise AssertionError(f"{ctx}: {int(bad.sum())} gradient entries out of tolerance, e.g. row {r[0]} "
                             f"index {i[0]}: gpu {g[r[0], i[0]]!r} oracle {ref[r[0], i[0]]!r} "
                             f"tol {tol[r[0], i[0]]!r}")
    return float((err / tol).max())
