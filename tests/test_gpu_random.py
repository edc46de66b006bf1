"""Seeded random cases through the HIP path, compared with the oracle. Each
case draws its shape (1-39 rows; a vocabulary of 1-63, 64-4095 or 4096-19999
entries, most not divisible by 8), its dtype pair, a row offset in the
handle, whether the rows start 2 elements past a 16-byte boundary (the
predicated path), next-token ids (some -1, some out of range) and a value
recipe: Gaussian, heavy-tailed, rounded to integers (many ties), nearly
identical rows, offsets of 1e4-3e4, a quantized row far flatter than the
base row (the row pass's second evaluation), 30 % of tokens masked at -1e4,
one dominant token, or a spread of thousands of nats, and a handle capacity
(the rows themselves, 2048 or 4096: the launch shapes of a bf16 pair). Every
case checks the per-token results, both summaries and the gradient; about a
third also the top-K stored form, its divergence and its gradient."""
import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import topk as otk
from tests.gpu_util import (check_summary_against_oracle, check_token_summary, compare_grad, compare_rows,
                            compare_token_rows, compare_topk_compress, compare_topk_grad, grad_to_f64,
                            run_gpu, say, topk_kl_tol)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 200
DTYPES = [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")]
RECIPES = ["gauss", "heavy", "ties", "close", "offset", "flat", "masked", "onehot", "huge"]


def _case(seed):
    g = np.random.default_rng(7000 + seed)
    n = int(g.integers(1, 40))
    v = int([g.integers(1, 64), g.integers(64, 4096), g.integers(4096, 20000)][int(g.integers(0, 3))])
    recipe = RECIPES[(seed // 4) % len(RECIPES)]
    if recipe == "gauss":
        zb = g.normal(0, 3, (n, v))
        zq = zb + g.normal(0, 0.2, (n, v))
    elif recipe == "heavy":
        zb = 3 * g.standard_t(3, (n, v))
        zq = zb * (1 + 0.02 * g.normal(size=(n, v))) + 0.1 * g.normal(size=(n, v))
    elif recipe == "ties":
        zb = np.round(g.normal(0, 2, (n, v)))
        zq = np.round(zb + g.normal(0, 0.5, (n, v)))
    elif recipe == "close":
        zb = g.normal(0, 4, (n, v))
        zq = zb + g.normal(0, 1e-3, (n, v))
    elif recipe == "offset":  # every logit shifted far from 0 (a bf16 side rounds to steps of 64-256)
        zb = float(g.choice([-3e4, -1e4, 1e4, 3e4])) + g.normal(0, 3, (n, v))
        zq = zb + g.normal(0, 0.2, (n, v))
    elif recipe == "flat":  # a quantized row far flatter than the base row
        zb = g.normal(0, 3, (n, v))
        zq = 0.05 * zb + g.normal(0, 0.05, (n, v))
    elif recipe == "masked":  # 30 % of the tokens at a large negative logit in both rows
        zb = g.normal(0, 3, (n, v))
        zq = zb + g.normal(0, 0.2, (n, v))
        m = g.random((n, v)) < 0.3
        zb[m] = -1e4
        zq[m] = -1e4
    elif recipe == "onehot":  # one token 60 nats above the rest; the quantized row's is another in 30 % of rows
        zb = g.normal(0, 1, (n, v))
        zq = zb + g.normal(0, 0.1, (n, v))
        hb = g.integers(0, v, n)
        hq = np.where(g.random(n) < 0.3, g.integers(0, v, n), hb)
        zb[np.arange(n), hb] += 60
        zq[np.arange(n), hq] += 60
    else:  # logits spread over thousands of nats
        zb = g.normal(0, 1e3, (n, v))
        zq = zb + g.normal(0, 10, (n, v))
    tokens = g.integers(-1, v + 1, n)
    return dict(n=n, v=v, dts=DTYPES[seed % 4], recipe=recipe, zb=zb, zq=zq, tokens=tokens,
                offset=int(g.integers(0, 5)), misalign=bool(g.integers(0, 2)), scale=float(g.normal()),
                gdt=["f32", "bf16"][int(g.integers(0, 2))], k=int(g.integers(1, min(v, 300) + 1)),
                topk=bool(g.integers(0, 3) == 0))


def _device(z, dt, misalign):
    t = torch.tensor(z, dtype=synth.torch_dtype(dt))
    if not misalign:
        return t.to(DEV)
    n, v = t.shape
    buf = torch.zeros(n * v + 8, dtype=t.dtype, device=DEV)
    view = buf[2:2 + n * v].view(n, v)  # 4 or 8 bytes past a 16-byte boundary
    view.copy_(t.to(DEV))
    return view


# seed 4339 (found by a sweep of 28,000 seeds): a collapsed bf16 base row
# at offset 1e4 whose merged waves carried rounding past the KL's tolerance
@pytest.mark.parametrize("seed", list(range(N_CASES)) + [4339])
def test_random_case_matches_oracle(seed):
    c = _case(seed)
    n, v, off = c["n"], c["v"], c["offset"]
    ctx = (f"seed {seed}: {n} x {v} {c['dts']} {c['recipe']} offset {off} misaligned {c['misalign']} "
           f"handle {[n + off, 2048, 4096][seed % 3]}")
    print(ctx, flush=True)
    b = _device(c["zb"], c["dts"][0], c["misalign"])
    q = _device(c["zq"], c["dts"][1], c["misalign"])
    nb, nq = synth.to_numpy_bits(b), synth.to_numpy_bits(q)
    o = oracle.rows(nb, nq)
    # handle capacity: the rows themselves, 2048 or 4096 rows -- the four-, two- and
    # one-wave-per-row shapes of a bf16 pair (an f32 side always runs four)
    cap = [n + off, 2048, 4096][seed % 3]
    with qqe.Evaluator(v, cap, c["dts"][0], c["dts"][1], device=DEV) as ev:
        g = run_gpu(b, q, row_offset=off, ev=ev, tokens=c["tokens"])
        (ks, ts), = ev.reduce_segments([off, off + n])
        compare_rows(g, o, ctx=ctx)
        check_summary_against_oracle(ks, o, ctx=ctx, strict_mean=False, row_base=off)
        tr, tb, tq, td = compare_token_rows(g, nb, nq, o, ctx=ctx)
        check_token_summary(ts, tr, tb, tq, td, g, ctx=ctx)
        grad = ev.grad(b, q, off, c["scale"], dtype=c["gdt"])
        torch.cuda.synchronize()
        compare_grad(grad_to_f64(grad), nb, nq, o, c["scale"], c["gdt"], ctx=ctx)
        if c["topk"]:
            k = c["k"]
            idx, logp, rest = ev.topk_compress(b, k)
            kl = torch.empty(n, dtype=torch.float32, device=DEV)
            match = torch.empty(n, dtype=torch.uint8, device=DEV)
            ev.rows_topk(idx, logp, rest, q, off, kl, match)
            torch.cuda.synchronize()
            lse_b = oracle.rows(nb, nb).lse_base
            gi, gl, gr = idx.cpu().numpy(), logp.cpu().numpy(), rest.cpu().numpy()
            compare_topk_compress(gi, gl, gr, otk.compress(nb, k, lse_b), lse_b, ctx=f"{ctx} k={k}")
            r = otk.kl_topk(otk.TopK(gi, gl, gr), nq, oracle.rows(nq, nq).lse_base)
            err = np.abs(kl.cpu().numpy().astype(np.float64) - r.kl)
            tol = topk_kl_tol(r.kl)
            assert (err <= tol).all(), f"{ctx} k={k}: coarsened KL"
            assert np.array_equal(match.cpu().numpy(), r.match), f"{ctx} k={k}: top-K match"
            gt = ev.grad_topk(idx, logp, q, off, c["scale"], dtype=c["gdt"])
            torch.cuda.synchronize()
            compare_topk_grad(grad_to_f64(gt), otk.TopK(gi, gl, gr), nq, oracle.rows(nq, nq).lse_base, c["scale"],
                              c["gdt"], ctx=f"{ctx} k={k}: top-K gradient")
    say(f"[random] {ctx} ok")
