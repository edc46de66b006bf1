"""GPU parity: the HIP path against the float64 oracle, element by element.

Oracle-sized cases run every row through the oracle (several wave-tiles per
row and ragged tails included). Full-size configurations run every row on the
GPU in the launch configuration the benchmark times and check every row
against the oracle (streamed to the host in row chunks), the summaries against
the oracle's, and the reduction against exact host arithmetic on the GPU's own
per-token values.
"""
import types

import numpy as np
import pytest
import torch

import oracle
import quantization_quality_eval_amd as qqe
import synth
from oracle import tokens as otok
from tests import pins
from tests.gpu_util import (assert_kl_close, check_summary_against_oracle, check_summary_properties,
                            check_token_summary, compare_rows, compare_token_rows, oracle_rows, run_gpu, say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gen(name, n_rows=None, vocab=None):
    cfg = synth.CONFIGS[name].scaled(n_rows=n_rows, vocab=vocab)
    b, q = synth.generate(cfg, device=DEV)
    return cfg, b, q


# ------------------------------------------------------------ oracle-sized ---

@pytest.mark.parametrize("name,n_rows,vocab", [
    ("c1", 64, 32000),            # the whole first configuration
    ("c2", 48, 151936),           # Qwen-sized rows: 296 wave-tiles + a 384-element tail
    ("c3", 32, 151936),           # mixed f32 / bf16, heavy tails
    ("c4", 40, 262144),           # 512 wave-tiles exactly, planted ties
    ("c5", 40, 151936),
    ("c2", 70, 151928),           # vocab % 512 != 0 with vector loads
    ("c4", 20, 4104),             # few wave-tiles per wave + tail
    ("c3", 24, 20000),
])
def test_parity_oracle_sized(name, n_rows, vocab):
    say(f"[parity] {name} n={n_rows} V={vocab}")
    cfg, b, q = _gen(name, n_rows, vocab)
    g = run_gpu(b, q)
    o = oracle_rows(b, q)
    abs_err, rel_err = compare_rows(g, o, ctx=f"{name} {n_rows}x{vocab}")
    full = (n_rows, vocab) == (synth.CONFIGS[name].n_rows, synth.CONFIGS[name].vocab)
    check_summary_against_oracle(g["summary"], o, ctx=name, strict_mean=full)
    check_summary_properties(g["summary"], g, ctx=name)
    say(f"[parity] {name}: max abs err {abs_err:.3e}, max rel err (above abs floor) {rel_err:.3e}")


def _ill_conditioned_rows(v, g):
    """Row pairs whose masses relative to their maxima differ by orders of
    magnitude (the row pass's fast form amplifies its fp32 rounding there and
    hands the rows to the second evaluation), and ordinary pairs beside them."""
    zb = g.normal(0, 3, (6, v))
    zq = np.empty_like(zb)
    zq[0] = 0.05 * zb[0] + g.normal(0, 0.05, v)       # quantized row far flatter (x >> 1)
    zq[1] = g.normal(0, 3, v)
    zb[1] = 0.05 * zq[1] + g.normal(0, 0.05, v)       # base row far flatter (x near -1)
    zb[2] = 1e4 + g.normal(0, 3, v)                   # at 1e4 a bfloat16 side collapses to a few values
    zq[2] = zb[2] + g.normal(0, 0.2, v)
    zq[3] = g.normal(0, 3, v)                         # independent rows
    zq[4] = zb[4] + g.normal(0, 0.2, v)               # ordinary pairs
    zq[5] = zb[5] + g.normal(0, 0.01, v)
    return zb, zq


@pytest.mark.parametrize("vocab", [4104, 151936])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("max_rows", [6, 2048, 4096])
def test_ill_conditioned_rows(vocab, dtypes, max_rows):
    """Per-token KL within 1e-5 relative / 1e-7 absolute, argmaxes and match
    bit-exact, also where the two distributions' peakedness differs by orders
    of magnitude; handles of 6, 2048 and 4096 rows select the four-, two- and
    one-wave-per-row shapes of the bf16 pair (an f32 side always runs four)."""
    zb, zq = _ill_conditioned_rows(vocab, np.random.default_rng(vocab))
    b = torch.tensor(zb, dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtypes[1]), device=DEV)
    with qqe.Evaluator(vocab, max_rows, dtypes[0], dtypes[1], device=DEV) as ev:
        g = run_gpu(b, q, ev=ev)
        summ = ev.reduce(b.shape[0])
    o = oracle_rows(b, q)
    ctx = f"ill-conditioned V={vocab} {dtypes} max_rows={max_rows}"
    abs_err, rel_err = compare_rows(g, o, ctx=ctx)
    check_summary_against_oracle(summ, o, ctx=ctx, strict_mean=False)
    f = g["flags"]
    say(f"[parity] {ctx}: KL {np.round(o.kl, 3).tolist()}, flags {f.tolist()}, "
        f"max rel err (above abs floor) {rel_err:.3e}")
    # the row pass hands both far-apart-peakedness rows to its float64 second
    # evaluation, each for its own reason: a quantized row far flatter than the
    # base row amplifies the sums' rounding (x = W_q / W_b - 1 ~ 10^3..10^4),
    # a base row far flatter than the quantized one leaves W_q / W_b ~ 10^-3
    assert f[0] & qqe.KLD_ROW_FLAG_AMPLIFIED, f"{ctx}: row 0 not taken again (flags {f[0]})"
    assert f[1] & qqe.KLD_ROW_FLAG_QUANT_MASS, f"{ctx}: row 1 not taken again (flags {f[1]})"


def _one_sided_rescale_rows(v, g):
    """Rows whose base running maximum jumps by 60 nats after a flat stretch
    while the quantized row's maximum does not jump there (its dominant token is
    elsewhere). The rescale at the jump moves the base mass accumulated so far
    (about one unit per flat element, so up to ~V) between the row pass's two
    sums, whose fp32 rounding then reaches the quant normaliser; the rows must be
    taken again. Rows 0-2, 4 and 5 put the base token in the row's last
    elements, which every launch shape visits after the flat stretch. Row 6 puts
    it mid-row: beyond its wave's first chunk at V = 151936, inside it at small
    vocabularies (both maxima are then set with no rescale and nothing is
    carried). Row 3 is the control: both dominant tokens at the same index and
    otherwise equal rows (KL exactly 0, nothing moved, nothing taken again)."""
    zb = np.zeros((7, v))
    zq = np.zeros((7, v))
    hb = [v - 1, v - 1, v - 3, v - 1, v - 1, v - 1, v // 2]   # base dominant token
    hq = [0, v // 2, v // 2 + 1, v - 1, 0, 3, 0]              # quant dominant token
    zq[4] = g.normal(0, 0.1, v)                               # quant noise beside a flat base
    zb[5] = g.normal(0, 0.2, v)                               # base not quite flat
    zq[5] = zb[5] + g.normal(0, 0.1, v)
    for r in range(7):
        zb[r, hb[r]] = zb[r].max() + 60.0
        zq[r, hq[r]] = zq[r].max() + 60.0
    return zb, zq


@pytest.mark.parametrize("vocab", [4104, 151936])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("max_rows", [7, 2048, 4096])
def test_one_sided_rescale_rows(vocab, dtypes, max_rows):
    """Regression case for far-apart dominant tokens with a large base mass at
    the jump (one-hot rows 60 nats above a flat rest, the two models' top
    tokens at different indices): per-token KL, both log-normalisers and both
    argmaxes against the oracle, and every such row flagged as carried. A
    7-row handle runs the four-waves-per-row shape, 2048 and 4096-row handles
    the two- and one-wave shapes of the bf16 pair."""
    zb, zq = _one_sided_rescale_rows(vocab, np.random.default_rng(vocab + 3))
    b = torch.tensor(zb, dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtypes[1]), device=DEV)
    ctx = f"one-sided rescale V={vocab} {dtypes} max_rows={max_rows}"
    say(f"[parity] {ctx}")
    with qqe.Evaluator(vocab, max_rows, dtypes[0], dtypes[1], device=DEV) as ev:
        g = run_gpu(b, q, ev=ev)
    o = oracle_rows(b, q)
    compare_rows(g, o, ctx=ctx)
    f = g["flags"]
    say(f"[parity] {ctx}: KL {np.round(o.kl, 3).tolist()}, flags {f.tolist()}")
    for r in (0, 1, 2, 4, 5) + ((6,) if vocab >= 65536 else ()):
        assert f[r] & qqe.KLD_ROW_FLAG_CARRIED, f"{ctx}: row {r} not taken again (flags {f[r]})"
    assert f[3] == 0 and g["kld"][3] == 0.0, f"{ctx}: control row flags {f[3]} KL {g['kld'][3]}"


def _collapsed_base_rows(v, g):
    """Base rows of 9984 everywhere but one token at 10048 (what a bf16 row of
    logits near 1e4 collapses to: bf16 steps are 64 there); quant rows of
    1e4 + N(0, 3^2) in float32 with their maximum at or near that token. In
    the four-waves-per-row shape three waves see a flat base, so their W
    grows to ~V/4 while C = sum(e - w) follows it down to about -W through
    every rise of their quant maximum; merging them into the row's shifts
    (base maximum 64 nats higher) scales that state down by e^-dq, and the
    rounding it carries is then large next to a KL of 0.1-3 although the
    quant normaliser, ~1e4, hides it. Found as seed 4339 of the random
    cases' recipe with offsets (one row 1.2x outside 1e-5 |KL| + 1e-7)."""
    zb = np.full((4, v), 9984.0)
    zq = 1e4 + g.normal(0, 3, (4, v))
    for r, (k, above) in enumerate([(764, 0.0), (5000, 1.0), (v - 270, 4.0), (100, 0.5)]):
        zb[r, k] = 10048.0
        zq[r, k] = zq[r].max() + above
    return zb, zq


@pytest.mark.parametrize("dtypes", [("bf16", "f32"), ("f32", "f32")])
def test_merged_waves_over_a_collapsed_base_row(dtypes):
    """Per-token KL within 1e-5 relative / 1e-7 absolute, argmaxes exact, and
    each row flagged as carrying moved mass (its KL bound, not its lse bound,
    is the one at risk)."""
    zb, zq = _collapsed_base_rows(12270, np.random.default_rng(11))
    b = torch.tensor(zb, dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtypes[1]), device=DEV)
    ctx = f"collapsed base rows {dtypes}"
    g = run_gpu(b, q)
    o = oracle_rows(b, q)
    f = g["flags"]
    err = np.abs(g["kld"].astype(np.float64) - o.kl)
    say(f"[parity] {ctx}: KL {np.round(o.kl, 4).tolist()}, |err| {err.tolist()}, flags {f.tolist()}")
    compare_rows(g, o, ctx=ctx)
    for r in range(4):
        assert f[r] & qqe.KLD_ROW_FLAG_CARRIED, f"{ctx}: row {r} not taken again (flags {f[r]})"


@pytest.mark.parametrize("vocab,max_rows,dtypes", [
    (262144, 2048, ("bf16", "bf16")), (262144, 4096, ("bf16", "bf16")),
    (1048576, 2048, ("bf16", "bf16")), (1048576, 4096, ("bf16", "bf16")),
    (4194304, 3, ("bf16", "bf16")), (4194304, 3, ("f32", "f32")), (4194304, 3, ("f32", "bf16"))])
@pytest.mark.parametrize("misaligned", [False, True])
def test_tied_rows_at_large_vocabularies(vocab, max_rows, dtypes, misaligned):
    """Integer-valued rows (a handful of distinct logits, each repeated
    thousands of times) of 2^18 and 2^20 tokens in the two- and one-wave
    shapes and of 2^22 tokens in the four-wave shape, aligned and through the
    predicated path: a lane then adds the same few values to its sums
    thousands of times, where fp32 rounding errors add up instead of
    averaging out; per-token KL, both log-normalisers and the argmaxes within
    the per-token bounds."""
    g = np.random.default_rng(vocab + max_rows)
    zb = np.round(g.normal(0, 2, (3, vocab)))
    zq = np.round(zb + g.normal(0, 0.5, (3, vocab)))
    b = torch.tensor(zb, dtype=synth.torch_dtype(dtypes[0]))
    q = torch.tensor(zq, dtype=synth.torch_dtype(dtypes[1]))
    if misaligned:  # 4 bytes past a 16-byte boundary: every element takes the predicated path
        bb = torch.zeros(3 * vocab + 8, dtype=b.dtype, device=DEV)
        qq = torch.zeros(3 * vocab + 8, dtype=q.dtype, device=DEV)
        k = 4 // b.element_size(), 4 // q.element_size()
        b_dev, q_dev = bb[k[0]:k[0] + 3 * vocab].view(3, vocab), qq[k[1]:k[1] + 3 * vocab].view(3, vocab)
        b_dev.copy_(b.to(DEV))
        q_dev.copy_(q.to(DEV))
    else:
        b_dev, q_dev = b.to(DEV), q.to(DEV)
    ctx = f"tied rows V={vocab} max_rows={max_rows} {dtypes} misaligned={misaligned}"
    say(f"[parity] {ctx}")
    with qqe.Evaluator(vocab, max_rows, dtypes[0], dtypes[1], device=DEV) as ev:
        gres = run_gpu(b_dev, q_dev, ev=ev)
    compare_rows(gres, oracle_rows(b_dev, q_dev), ctx=ctx)


# (vocab, handle rows, dtypes): a vocabulary divisible by 8 streams by
# 16-byte tiles, an odd one takes the predicated path for every element
@pytest.mark.parametrize("vocab,max_rows,dtypes", [
    (2 ** 31 - 8, 4096, ("bf16", "bf16")), (2 ** 31 - 8, 2, ("bf16", "bf16")),
    (2 ** 31 - 8, 2, ("f32", "f32")), (2 ** 31 - 1, 2, ("bf16", "bf16")),
    (2 ** 28 + 1, 4096, ("bf16", "bf16"))])
def test_flat_rows_at_the_vocabulary_limit(vocab, max_rows, dtypes):
    """Rows flat but for a few tokens, up to the largest vocabulary the library
    accepts (2^31 - 1). A token raised at the very start sets the running
    maxima there, so every later term of a row's sums is the same number,
    e^-3 (base) or e^-2.5 (quantized) -- the case where float32 partial sums
    drift furthest, their roundings all going one way. The row maxima sit
    near the end (indices near 2^31): on the same token in row 0, on
    neighbouring tokens in row 1. Checked against closed forms, in the
    one-wave and four-wave shapes (the closed forms are pinned against the
    oracle in tests/pins.py)."""
    rows_b = [{0: 3.0, vocab - 2: 20.0}, {0: 3.0, vocab - 2: 20.0}]  # exact in bfloat16
    rows_q = [{0: 2.5, vocab - 2: 18.0}, {0: 2.5, vocab - 3: 18.0}]
    ctx = f"flat rows V={vocab} max_rows={max_rows} {dtypes}"
    say(f"[parity] {ctx}")
    b = torch.zeros((2, vocab), dtype=synth.torch_dtype(dtypes[0]), device=DEV)
    q = torch.zeros((2, vocab), dtype=synth.torch_dtype(dtypes[1]), device=DEV)
    for r in range(2):
        for i, v in rows_b[r].items():
            b[r, i] = v
        for i, v in rows_q[r].items():
            q[r, i] = v
    with qqe.Evaluator(vocab, max_rows, dtypes[0], dtypes[1], device=DEV) as ev:
        g = run_gpu(b, q, ev=ev)
    del b, q
    torch.cuda.empty_cache()
    forms = [pins.flat_rows_closed_form(vocab, rb, rq) for rb, rq in zip(rows_b, rows_q)]
    want = types.SimpleNamespace(
        kl=np.array([f[0] for f in forms]), lse_base=np.array([f[1] for f in forms]),
        lse_quant=np.array([f[2] for f in forms]),
        argmax_base=np.array([vocab - 2, vocab - 2], np.int64),
        argmax_quant=np.array([vocab - 2, vocab - 3], np.int64), match=np.array([1, 0], np.uint8))
    say(f"[parity] {ctx}: KL {g['kld'].tolist()} vs {want.kl.tolist()}, lse_b {g['lse_b'].tolist()} vs "
        f"{want.lse_base.tolist()}, lse_q {g['lse_q'].tolist()} vs {want.lse_quant.tolist()}, "
        f"flags {g['flags'].tolist()}")
    compare_rows(g, want, ctx=ctx)


def test_planted_rows_behave_as_planted():
    cfg, b, q = _gen("c2", 100, 151936)
    plan = synth.row_plan(cfg)
    g = run_gpu(b, q)
    moved = plan.moved[:100]
    assert moved.any()
    assert np.all(g["match"][moved] == 0) and np.all(g["match"][~moved] == 1)
    assert np.array_equal(g["ab"], plan.peak[:100])
    cfg, b, q = _gen("c4", 60, 8192)
    plan = synth.row_plan(cfg)
    g = run_gpu(b, q)
    t = plan.tie
    assert t.any()
    assert np.array_equal(g["ab"][t], plan.tie_i[t]) and np.array_equal(g["aq"][t], plan.tie_i[t])


# ------------------------------------------------------------- edge shapes ---

@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 8, 65, 511, 512, 513, 1000, 4096 + 8, 32768 + 100])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_edge_vocab_sizes(vocab, dtypes):
    say(f"[edge] V={vocab} {dtypes}")
    g0 = torch.Generator(device=DEV).manual_seed(vocab * 7 + len(dtypes[0]))
    n = 65
    zb = (3.0 * torch.randn(n, vocab, generator=g0, device=DEV)).to(synth.torch_dtype(dtypes[0]))
    zq = (zb.float() + 0.3 * torch.randn(n, vocab, generator=g0, device=DEV)).to(synth.torch_dtype(dtypes[1]))
    g = run_gpu(zb, zq)
    o = oracle_rows(zb, zq)
    compare_rows(g, o, ctx=f"V={vocab} {dtypes}")
    check_summary_against_oracle(g["summary"], o, ctx=f"V={vocab}", strict_mean=False)


@pytest.mark.parametrize("n_rows", [1, 63, 64, 65, 1500, 2500, 4100])
def test_edge_row_counts(n_rows):
    # 1500, 2500 and 4100 rows select the four-, two- and one-wave-per-row
    # launch shapes
    cfg, b, q = _gen("c5", n_rows, 2048 + 72)
    g = run_gpu(b, q)
    o = oracle_rows(b, q)
    compare_rows(g, o, ctx=f"n={n_rows}")
    check_summary_against_oracle(g["summary"], o, ctx=f"n={n_rows}", strict_mean=False)


def test_unaligned_row_pointers_take_the_predicated_path():
    cfg, b, q = _gen("c2", 9, 4097)
    full_b = torch.empty(9 * 4097 + 1, dtype=b.dtype, device=DEV)
    full_q = torch.empty(9 * 4097 + 3, dtype=q.dtype, device=DEV)
    vb = full_b[1:].view(9, 4097)
    vq = full_q[3:].view(9, 4097)
    vb.copy_(b)
    vq.copy_(q)
    assert vb.data_ptr() % 16 != 0
    g = run_gpu(vb, vq)
    o = oracle_rows(b, q)
    compare_rows(g, o, ctx="unaligned")
    # same bytes through aligned storage with a vocab that allows vector loads
    cfg, b, q = _gen("c2", 9, 4096)
    full_b = torch.empty(9 * 4096 + 8, dtype=b.dtype, device=DEV)
    vb = full_b[8:].view(9, 4096)           # 16-byte aligned offset
    vb.copy_(b)
    compare_rows(run_gpu(vb, q), oracle_rows(b, q), ctx="offset-aligned")


def _rows_from(zb64, zq64, bt="f32", qt="f32"):
    zb = torch.tensor(zb64, dtype=torch.float64).to(synth.torch_dtype(bt)).to(DEV)
    zq = torch.tensor(zq64, dtype=torch.float64).to(synth.torch_dtype(qt)).to(DEV)
    return zb, zq


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ties_zeros_and_degenerate_rows(dt):
    v = 1536 + 40
    rng = np.random.default_rng(5)
    zb = rng.normal(0, 2, (14, v))
    zq = zb + rng.normal(0, 0.2, (14, v))
    zb[0, :] = 1.25
    zq[0, :] = 1.25                         # constant rows: KL 0, argmax 0
    zb[1, [0, v - 1]] = 30.0                # tie at both ends
    zq[1, [v - 1, 7]] = 30.0
    zb[2, :] = 0.0
    zb[2, 100] = -0.0                       # +0 / -0 everywhere: a tie at index 0
    zq[2, :] = -0.0
    zb[3, [513, 514, 1030]] = 12.0          # ties across lanes / wave-tiles
    zq[3, [1030, 514]] = 12.0
    zq[4] = zb[4]                           # identical rows: KL exactly 0
    zb[5, v - 3] = 50.0                     # max in the predicated tail
    zq[5, v - 40] = 50.0
    zq[6, 77] = zq[6].max() + 120.0         # quant peak far above the quant at the base argmax
    zb[7] *= 40.0                           # large-magnitude logits
    zq[7] = zb[7] + rng.normal(0, 1.0, v)
    zb[8, 3] = zb[8, 3 + 512] = zb[8, 3 + 1024] = 9.0   # same lane position, three wave-tiles
    # shifts thousands of nats apart between waves / within a wave (heavy tails)
    zb[9, 5] = 3000.0
    zq[9, 5] = 2700.0                       # merge: base and quant shifts move by ~3000 and ~2700
    zb[10, 900] = 5000.0
    zq[10, 1300] = 4000.0                   # different peaks, divergence ~ thousands of nats
    zq[11, 10] = 2500.0                     # only the quant row has a huge logit
    zb[12, :] = 0.0                         # subnormal maxima (below 2^-126), tied in base
    zb[12, [300, 700]] = 5e-40
    zq[12, :] = -0.0
    zq[12, 1500] = 3e-40
    zb[13, :] = -1e-39                      # all-negative subnormal row, one zero
    zb[13, 1000] = -0.0
    zq[13, :] = -2e-39
    zq[13, 5] = -1e-39
    b, q = _rows_from(zb, zq, dt, dt)
    g = run_gpu(b, q)
    o = oracle_rows(b, q)
    compare_rows(g, o, ctx=f"degenerate {dt}")
    assert g["kld"][0] == 0.0 and g["kld"][4] == 0.0
    assert g["ab"][1] == 0 and g["aq"][1] == 7 and g["ab"][2] == 0 and g["aq"][2] == 0
    assert g["ab"][3] == 513 and g["aq"][3] == 514 and g["ab"][8] == 3
    assert np.all(np.isfinite(g["kld"]))
    assert g["ab"][9] == 5 and g["ab"][10] == 900 and g["aq"][10] == 1300 and g["aq"][11] == 10
    assert g["ab"][12] == 300 and g["aq"][12] == 1500 and g["ab"][13] == 1000 and g["aq"][13] == 5


# ------------------------------------------------- determinism and streams ---

def test_bit_reproducible_and_chunking_invariant():
    cfg, b, q = _gen("c5", 512, 151936)
    n = b.shape[0]
    g1 = run_gpu(b, q)
    g2 = run_gpu(b, q)
    for k in ("kld", "match", "ab", "aq", "lse_b", "lse_q"):
        assert np.array_equal(g1[k], g2[k]), k
    # 8 chunks, alternating two streams, into one handle; one reduce
    ev = qqe.Evaluator(151936, n, "bf16", "bf16", device=DEV)
    kld = torch.empty(n, dtype=torch.float32, device=DEV)
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    step = n // 8
    for i in range(8):
        s = streams[i % 2]
        with torch.cuda.stream(s):
            ev.rows(b[i * step:(i + 1) * step], q[i * step:(i + 1) * step], i * step,
                    kld_out=kld[i * step:(i + 1) * step], stream=s)
    summ = ev.reduce(n)
    torch.cuda.synchronize()
    assert np.array_equal(kld.cpu().numpy(), g1["kld"])
    assert summ == g1["summary"]
    # chunks in reverse order on the default stream
    ev2 = qqe.Evaluator(151936, n, "bf16", "bf16", device=DEV)
    for i in reversed(range(8)):
        ev2.rows(b[i * step:(i + 1) * step], q[i * step:(i + 1) * step], i * step)
    assert ev2.reduce(n) == g1["summary"]
    ev.close()
    ev2.close()


@pytest.mark.parametrize("n_rows,vocab", [(6, 151936), (300, 32000)])
def test_timed_rows_match_plain_rows(n_rows, vocab):
    """kld_eval_rows_timed: the row kernel's launch records the start / stop
    events itself; the per-token results and the summary are bit-identical to
    kld_eval_rows', the elapsed time is positive, and the same events can be
    passed again."""
    _, b, q = _gen("c2", n_rows, vocab)
    g = run_gpu(b, q)
    ev = qqe.Evaluator(vocab, n_rows, "bf16", "bf16", device=DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(2):
        kld = torch.empty(n_rows, dtype=torch.float32, device=DEV)
        match = torch.empty(n_rows, dtype=torch.uint8, device=DEV)
        ab = torch.empty(n_rows, dtype=torch.int32, device=DEV)
        aq = torch.empty(n_rows, dtype=torch.int32, device=DEV)
        ev.rows(b, q, 0, kld, match, ab, aq, start_event=e0, stop_event=e1)
        e1.synchronize()
        assert e0.elapsed_time(e1) > 0
        assert np.array_equal(kld.cpu().numpy(), g["kld"])
        assert np.array_equal(match.cpu().numpy(), g["match"])
        assert np.array_equal(ab.cpu().numpy(), g["ab"]) and np.array_equal(aq.cpu().numpy(), g["aq"])
        assert ev.reduce(n_rows) == g["summary"]
    with pytest.raises(ValueError):
        ev.rows(b, q, 0, start_event=e0, tokens=torch.zeros(n_rows, dtype=torch.int32, device=DEV))
    ev.close()


def test_reduction_paths_agree_bit_for_bit():
    """The one-launch reduction (kld_eval_reduce over [0, n), and the
    asynchronous kld_eval_reduce_async into pinned host memory or device
    memory) and the two-level table-driven one (a segment list whose first
    segment is [0, n)) give the same bits, for several row counts (one tile,
    a ragged tile, several tiles), with rows fed in chunks on two streams."""
    v = 4104
    cfg, b, q = _gen("c2", 5000, v)
    n = b.shape[0]
    with qqe.Evaluator(v, n, "bf16", "bf16", device=DEV) as ev:
        streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        step = 1250
        for i in range(4):
            s = streams[i % 2]
            with torch.cuda.stream(s):
                ev.rows(b[i * step:(i + 1) * step], q[i * step:(i + 1) * step], i * step, stream=s)
        for m in (1, 1000, 1024, 1025, 3333, n):
            pinned = ev.reduce_async(m)                     # ordered after both streams' rows
            on_dev = ev.reduce_async(m, out=torch.empty(64, dtype=torch.uint8, device=DEV))
            torch.cuda.synchronize()
            a, d = qqe.summary_from_bytes(pinned), qqe.summary_from_bytes(on_dev)
            blocking = ev.reduce(m)
            (two_level, _), (empty, _) = ev.reduce_segments([0, m, m])
            assert empty.n_rows == 0
            for x in (a, d, two_level):
                assert x == blocking, f"{m} rows: {x} vs {blocking}"
            assert blocking.n_rows == m
        say(f"[reduce] one-launch, asynchronous and two-level reductions identical; mean {blocking.kld_mean:.8g}")
        with pytest.raises(ValueError):
            ev.reduce_async(n, out=torch.empty(64, dtype=torch.uint8))   # host memory the device cannot write
        with pytest.raises(qqe.KldEvalError) as e:
            ev.reduce_async(0)
        assert e.value.status == qqe.KLD_ERR_EMPTY


def test_output_guard_bands_untouched():
    cfg, b, q = _gen("c2", 33, 8192)
    n, pad = 33, 64
    kld = torch.full((n + 2 * pad,), 7.5, dtype=torch.float32, device=DEV)
    match = torch.full((n + 2 * pad,), 0xAB, dtype=torch.uint8, device=DEV)
    ab = torch.full((n + 2 * pad,), -77, dtype=torch.int32, device=DEV)
    aq = torch.full((n + 2 * pad,), -77, dtype=torch.int32, device=DEV)
    with qqe.Evaluator(8192, n + 10, "bf16", "bf16", device=DEV) as ev:
        ev.rows(b, q, 10, kld[pad:pad + n], match[pad:pad + n], ab[pad:pad + n], aq[pad:pad + n])
        torch.cuda.synchronize()
    for t, fillv in ((kld, 7.5), (match, 0xAB), (ab, -77), (aq, -77)):
        assert (t[:pad] == fillv).all() and (t[pad + n:] == fillv).all()
        assert not (t[pad:pad + n] == fillv).all()


# --------------------------------------------------------------- API errors ---

def test_api_errors_with_device(monkeypatch):
    with qqe.Evaluator(1024, 16, "f32", "f32", device=DEV) as ev:
        b = torch.randn(8, 1024, device=DEV)
        with pytest.raises(qqe.KldEvalError) as e:
            ev.rows(b, b, row_offset=9)
        assert e.value.status == qqe.KLD_ERR_RANGE
        with pytest.raises(qqe.KldEvalError) as e:
            ev.reduce(0)
        assert e.value.status == qqe.KLD_ERR_EMPTY
        with pytest.raises(qqe.KldEvalError) as e:
            ev.reduce(17)
        assert e.value.status == qqe.KLD_ERR_RANGE
        with pytest.raises(TypeError):
            ev.rows(b.bfloat16(), b)
        # outputs on the host are refused before any launch (a host address
        # would otherwise reach the kernel)
        with pytest.raises(ValueError):
            ev.rows(b, b, 0, torch.empty(8))
        with pytest.raises(ValueError):
            ev.copy_lse(0, 8, torch.empty(8))
        with pytest.raises(ValueError):
            ev.row_flags(0, 8, out=torch.empty(8, dtype=torch.uint8))
        ev.rows(b[:0], b[:0])                       # zero rows: no-op
        h = ev.handle
    with pytest.raises(qqe.KldEvalError) as e:      # use after destroy
        qqe.kld_eval_rows(h, b.data_ptr(), b.data_ptr(), 8, 0)
    assert e.value.status == qqe.KLD_ERR_BAD_HANDLE
    monkeypatch.setenv("KLD_EVAL_FAIL_ALLOC", "1")
    with pytest.raises(qqe.KldEvalError) as e:
        qqe.Evaluator(1024, 16, "f32", "f32", device=DEV)
    assert e.value.status == qqe.KLD_ERR_OUT_OF_MEMORY


# ------------------------------------------------ full-size configurations ---

def _full_check(name, b, q, g, chunk=2048):
    """Every row against the oracle, streamed to the host in row chunks; with
    token outputs in ``g`` the token-conditioned values and summary too."""
    n = b.shape[0]
    kl = np.empty(n)
    match = np.empty(n, np.uint8)
    with_tokens = "lpb" in g
    parts = []
    worst_abs = 0.0
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        nb = synth.to_numpy_bits(b[r0:r0 + rows.size])
        nq = synth.to_numpy_bits(q[r0:r0 + rows.size])
        o = oracle.rows(nb, nq)
        abs_err, _ = compare_rows(g, o, rows, ctx=f"{name} rows {r0}..{r0 + rows.size}")
        if with_tokens:
            parts.append(compare_token_rows(g, nb, nq, o, rows, ctx=f"{name} rows {r0}..{r0 + rows.size}"))
        worst_abs = max(worst_abs, abs_err)
        kl[rows] = o.kl
        match[rows] = o.match
        if r0 % (8 * chunk) == 0:
            say(f"[full] {name}: rows < {r0 + rows.size} ok")
    whole = oracle.RowResults(kl, None, None, match, None, None)
    check_summary_against_oracle(g["summary"], whole, ctx=name)
    check_summary_properties(g["summary"], g, ctx=name)
    if with_tokens:
        tr = otok.TokenRows(*(np.concatenate([getattr(p[0], f) for p in parts])
                              for f in ("logp_base", "logp_quant", "dp", "state")))
        tb, tq, td = (np.concatenate([p[i] for p in parts]) for i in (1, 2, 3))
        check_token_summary(g["token_summary"], tr, tb, tq, td, g, ctx=name)
    s = g["summary"]
    say(f"[full] {name}: all {n} rows ok; max abs err {worst_abs:.3e}; mean {s.kld_mean:.8g} "
        f"max {s.kld_max:.6g} (row {s.kld_max_row}) same-top1 {s.same_top1:.6f}")


@pytest.mark.slow
def test_full_c2():
    cfg, b, q = _gen("c2")
    g = run_gpu(b, q, tokens=synth.tokens(cfg))
    plan = synth.row_plan(cfg)
    _full_check("c2", b, q, g)
    assert g["summary"].n_match == cfg.n_rows - int(plan.moved.sum())
    # the row pass's float64 second evaluation is for ill-conditioned rows; no
    # row of this workload is one, so none pays for it
    assert not g["flags"].any(), f"c2: {int((g['flags'] != 0).sum())} rows taken again"
    del b, q
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_full_c4():
    cfg, b, q = _gen("c4")
    g = run_gpu(b, q, tokens=synth.tokens(cfg))
    plan = synth.row_plan(cfg)
    ties = np.nonzero(plan.tie)[0]
    assert np.array_equal(g["ab"][ties], plan.tie_i[ties])
    assert np.array_equal(g["aq"][ties], plan.tie_i[ties])
    _full_check("c4", b, q, g)
    say(f"[full] c4: {int((g['flags'] != 0).sum())} rows taken again in float64")
    del b, q
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_full_c3():
    cfg = synth.CONFIGS["c3"]
    b, q = synth.generate(cfg, device=DEV)
    g = run_gpu(b, q, tokens=synth.tokens(cfg))
    _full_check("c3", b, q, g)
    say(f"[full] c3: {int((g['flags'] != 0).sum())} rows taken again in float64")
    del b, q
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_full_c5_chunked_two_streams():
    cfg = synth.CONFIGS["c5"]
    n, step = cfg.n_rows, cfg.chunk_rows
    b = torch.empty((n, cfg.vocab), dtype=torch.bfloat16, device=DEV)
    q = torch.empty_like(b)
    plan = synth.row_plan(cfg)
    for i in range(n // step):
        synth.fill(cfg, b[i * step:(i + 1) * step], q[i * step:(i + 1) * step], i * step, plan)
    kld = torch.empty(n, dtype=torch.float32, device=DEV)
    match = torch.empty(n, dtype=torch.uint8, device=DEV)
    ab = torch.empty(n, dtype=torch.int32, device=DEV)
    aq = torch.empty(n, dtype=torch.int32, device=DEV)
    tokens = synth.tokens(cfg)
    tok = torch.as_tensor(tokens, device=DEV)
    lpb, lpq, dp = (torch.empty(n, dtype=torch.float32, device=DEV) for _ in range(3))
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    with qqe.Evaluator(cfg.vocab, n, "bf16", "bf16", device=DEV) as ev:
        for i in range(n // step):
            s = streams[i % 2]
            sl = slice(i * step, (i + 1) * step)
            with torch.cuda.stream(s):
                ev.rows(b[sl], q[sl], i * step, kld[sl], match[sl], ab[sl], aq[sl], stream=s, tokens=tok[sl],
                        logp_base_out=lpb[sl], logp_quant_out=lpq[sl], dp_out=dp[sl])
        summ = ev.reduce(n)
        tsum = ev.reduce_tokens(n)
        lse_b = torch.empty(n, dtype=torch.float32, device=DEV)
        lse_q = torch.empty(n, dtype=torch.float32, device=DEV)
        ev.copy_lse(0, n, lse_b, lse_q)
        flags = ev.row_flags(0, n)
        torch.cuda.synchronize()
    assert not flags.any(), f"c5: {int((flags != 0).sum())} rows taken again"
    g = dict(kld=kld.cpu().numpy(), match=match.cpu().numpy(), ab=ab.cpu().numpy(), aq=aq.cpu().numpy(),
             lse_b=lse_b.cpu().numpy(), lse_q=lse_q.cpu().numpy(), summary=summ, lpb=lpb.cpu().numpy(),
             lpq=lpq.cpu().numpy(), dp=dp.cpu().numpy(), tokens=tokens, token_summary=tsum)
    _full_check("c5", b, q, g)
    del b, q
    torch.cuda.empty_cache()
