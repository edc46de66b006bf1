"""Seeded generators: determinism, block addressing, planted structure (no GPU)."""
import numpy as np
import torch

import synth


def test_same_seed_same_bytes():
    cfg = synth.CONFIGS["c1"].scaled(n_rows=8, vocab=1000)
    a = synth.generate(cfg)
    b = synth.generate(cfg)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_row_ranges_equal_whole_generation():
    cfg = synth.CONFIGS["c5"].scaled(n_rows=3 * synth.BLOCK_ROWS // 2, vocab=300)
    whole = synth.generate(cfg)
    r0, r1 = 100, 350            # crosses a block boundary
    part = synth.generate(cfg, r0, r1)
    assert torch.equal(whole[0][r0:r1], part[0]) and torch.equal(whole[1][r0:r1], part[1])


def test_dtypes_and_shapes():
    for name, cfg in synth.CONFIGS.items():
        small = cfg.scaled(n_rows=4, vocab=512)
        b, q = synth.generate(small)
        assert b.shape == q.shape == (4, 512)
        assert b.dtype == synth.torch_dtype(cfg.base_dtype)
        assert q.dtype == synth.torch_dtype(cfg.quant_dtype)
        assert torch.isfinite(b.float()).all() and torch.isfinite(q.float()).all()


def test_peak_config_plants_peak_and_moves_two_percent():
    cfg = synth.CONFIGS["c2"].scaled(n_rows=300, vocab=2000)
    plan = synth.row_plan(cfg)
    assert plan.moved.sum() == int(0.02 * 300)
    b, q = synth.generate(cfg)
    bf, qf = b.float(), q.float()
    rows = torch.arange(300)
    peak = torch.as_tensor(plan.peak)
    # the planted base peak is the row's strict maximum, >= 12 nats above the rest
    top2 = bf.topk(2, dim=1).values
    assert torch.equal(bf.argmax(dim=1), peak)
    assert (top2[:, 0] - top2[:, 1] >= 11.5).all()
    moved = torch.as_tensor(plan.moved)
    qpeak = qf.argmax(dim=1)
    assert torch.equal(qpeak[~moved], peak[~moved])
    assert torch.equal(qpeak[moved], torch.as_tensor(plan.moved_to)[moved])
    assert (qf[rows, peak] < qf.max(dim=1).values)[moved].all()


def test_tie_config_plants_exact_ties_in_both_rows():
    cfg = synth.CONFIGS["c4"].scaled(n_rows=90, vocab=1500)
    plan = synth.row_plan(cfg)
    assert plan.tie.sum() == 9
    b, q = synth.generate(cfg)
    bf, qf = b.float(), q.float()
    for r in np.nonzero(plan.tie)[0]:
        i, j = plan.tie_i[r], plan.tie_j[r]
        assert i < j
        assert bf[r, i] == bf[r, j] == bf[r].max()
        assert qf[r, i] == qf[r, j] == qf[r].max()
        assert (bf[r] == bf[r].max()).sum() == 2


def test_student_config_has_heavy_tails():
    cfg = synth.CONFIGS["c3"].scaled(n_rows=8, vocab=20000)
    b, q = synth.generate(cfg)
    assert b.dtype == torch.float32 and q.dtype == torch.bfloat16
    # Student-t(3) * 3 reaches far beyond a Gaussian of similar scale
    assert b.abs().max() > 40


def test_token_ids_are_seeded_in_range_and_mark_context_ends():
    for name in ("c1", "c2", "c4"):
        cfg = synth.CONFIGS[name]
        t = synth.tokens(cfg)
        assert t.dtype == np.int32 and t.shape == (cfg.n_rows,)
        assert np.array_equal(t, synth.tokens(cfg))
        ends = (np.arange(cfg.n_rows) % synth.CONTEXT_ROWS) == synth.CONTEXT_ROWS - 1
        assert np.all(t[ends] == -1) and np.all((t[~ends] >= 0) & (t[~ends] < cfg.vocab))
        assert np.array_equal(synth.tokens(cfg, 10, 40), t[10:40])
    cfg = synth.CONFIGS["c2"]
    plan = synth.row_plan(cfg)
    frac = np.mean(synth.tokens(cfg)[:-1] == plan.peak[:-1])
    assert 0.45 < frac < 0.55
