"""Seeded synthetic logit generators shared by the tests and the benchmark.

This module only draws random numbers and lays them out as logit rows; it holds
none of the comparison's arithmetic (no softmax, no divergence, no argmax of the
final rows). Both the HIP path and the oracle read the bytes it produces: the
bytes are the contract, not the random stream, so the same seed may give other
bytes on another device type.

The rows stand in for the pages' workloads, which cannot be reproduced here
(no models, no evaluation text): a Qwen-class vocabulary of 151936 entries
scored over 8192-token contexts ("Qwen3.6 27B Quantization Benchmark",
"Measurement method"), and many fixed-length chunks per domain (GSQ-RCO model
card, "Quality"). Each configuration below states its value distribution.

Randomness:
* bulk normals come from ``torch.randn`` with a ``torch.Generator`` seeded per
  block of ``BLOCK_ROWS`` rows, so any block can be regenerated on its own;
* the small per-row choices (planted peak positions, which rows get a moved
  peak or a tie, the partner index) come from NumPy's PCG64 seeded by
  ``SeedSequence([seed, config id, stream id])``, identical on every device.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

BLOCK_ROWS = 256


@dataclass(frozen=True)
class Config:
    name: str
    cid: int
    n_rows: int
    vocab: int
    base_dtype: str   # "f32" | "bf16"
    quant_dtype: str  # "f32" | "bf16"
    kind: str         # generator recipe, see _fill_block
    seed: int = 0
    chunk_rows: int = 0   # >0: the workload is fed in chunks of this many rows
    streams: int = 1
    params: dict = field(default_factory=dict)

    @property
    def bytes_per_row(self) -> int:
        return self.vocab * (_size(self.base_dtype) + _size(self.quant_dtype))

    @property
    def total_bytes(self) -> int:
        return self.n_rows * self.bytes_per_row

    def scaled(self, n_rows: int | None = None, vocab: int | None = None) -> "Config":
        """Same recipe at another size (for oracle-sized parity cases)."""
        return replace(self, n_rows=n_rows or self.n_rows, vocab=vocab or self.vocab)


def _size(dt: str) -> int:
    return 4 if dt == "f32" else 2


def torch_dtype(dt: str):
    return torch.float32 if dt == "f32" else torch.bfloat16


CONFIGS = {
    # 64 x 32000 fp32, base N(0, 3^2), quant = base + N(0, 0.1^2)
    "c1": Config("c1", 1, 64, 32000, "f32", "f32", "gauss",
                 params=dict(base_sigma=3.0, noise_sigma=0.1)),
    # one 8192-token context, V=151936 bf16, base N(0, 4^2) with one planted
    # peak per row 12 nats above the row's natural maximum, quant = base +
    # N(0, 0.05^2), and 2% of rows with the quant's peak moved elsewhere
    "c2": Config("c2", 2, 8192, 151936, "bf16", "bf16", "peak",
                 params=dict(base_sigma=4.0, noise_sigma=0.05, peak_margin=12.0,
                             moved_frac=0.02)),
    # 8 contexts of 8192, fp32 base vs bf16 quant, Student-t(3) scale 3 base,
    # quant = base * (1 + N(0, 0.02^2)) + N(0, 0.1^2)
    "c3": Config("c3", 3, 65536, 151936, "f32", "bf16", "student",
                 params=dict(scale=3.0, nu=3, mult_sigma=0.02, add_sigma=0.1)),
    # V=262144 bf16, base N(0, 4^2), quant noise sigma by row thirds
    # {0.01, 0.1, 0.5}, 10% of rows with an exact two-way tie for the maximum
    "c4": Config("c4", 4, 16384, 262144, "bf16", "bf16", "ties",
                 params=dict(base_sigma=4.0, sigmas=(0.01, 0.1, 0.5), tie_frac=0.1)),
    # 16 contexts of 8192, V=151936 bf16, base N(0, 4^2), quant = base +
    # N(0, 0.2^2), fed as 8 chunks of 16384 rows alternating two streams
    "c5": Config("c5", 5, 131072, 151936, "bf16", "bf16", "gauss",
                 chunk_rows=16384, streams=2,
                 params=dict(base_sigma=4.0, noise_sigma=0.2)),
}


def _block_seed(cfg: Config, tensor_id: int, block: int) -> int:
    ss = np.random.SeedSequence([cfg.seed, cfg.cid, tensor_id, block])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _rng(cfg: Config, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, cfg.cid, 1000 + stream])))


@dataclass
class RowPlan:
    """Per-row choices for the whole configuration (small, host-side)."""
    peak: np.ndarray | None = None       # planted peak index per row
    moved: np.ndarray | None = None      # bool per row: quant peak moved
    moved_to: np.ndarray | None = None   # index the quant peak moves to
    tie: np.ndarray | None = None        # bool per row: planted two-way tie
    tie_i: np.ndarray | None = None      # lower tied index
    tie_j: np.ndarray | None = None      # higher tied index


def row_plan(cfg: Config) -> RowPlan:
    n, v = cfg.n_rows, cfg.vocab
    if cfg.kind == "peak":
        g = _rng(cfg, 0)
        peak = g.integers(0, v, size=n)
        n_moved = int(np.floor(cfg.params["moved_frac"] * n))
        moved = np.zeros(n, bool)
        moved[g.permutation(n)[:n_moved]] = True
        off = g.integers(1, v, size=n) if v > 1 else np.zeros(n, np.int64)
        moved_to = (peak + off) % v          # uniform over the other indices
        return RowPlan(peak=peak, moved=moved, moved_to=moved_to)
    if cfg.kind == "ties":
        g = _rng(cfg, 0)
        n_tie = int(np.floor(cfg.params["tie_frac"] * n))
        tie = np.zeros(n, bool)
        tie[g.permutation(n)[:n_tie]] = True
        a = g.integers(0, v, size=n)
        off = g.integers(1, v, size=n) if v > 1 else np.zeros(n, np.int64)
        b = (a + off) % v
        return RowPlan(tie=tie, tie_i=np.minimum(a, b), tie_j=np.maximum(a, b))
    return RowPlan()


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _fill_block(cfg: Config, plan: RowPlan, r0: int, r1: int, device):
    """Generate rows [r0, r1) of one block; returns (base, quant) on device."""
    blk = r0 // BLOCK_ROWS
    shape = (r1 - r0, cfg.vocab)
    p = cfg.params
    bt, qt = torch_dtype(cfg.base_dtype), torch_dtype(cfg.quant_dtype)
    rows = torch.arange(r0, r1, device=device)
    if cfg.kind == "gauss":
        zb = (p["base_sigma"] * _randn(shape, _block_seed(cfg, 0, blk), device)).to(bt)
        zq = (zb.float() + p["noise_sigma"] * _randn(shape, _block_seed(cfg, 1, blk), device)).to(qt)
        return zb, zq
    if cfg.kind == "peak":
        zb32 = p["base_sigma"] * _randn(shape, _block_seed(cfg, 0, blk), device)
        k = torch.as_tensor(plan.peak[r0:r1], device=device)
        top = zb32.max(dim=1).values
        zb32[torch.arange(r1 - r0, device=device), k] = top + p["peak_margin"]
        zb = zb32.to(bt)
        zq = (zb.float() + p["noise_sigma"] * _randn(shape, _block_seed(cfg, 1, blk), device)).to(qt)
        mv = np.nonzero(plan.moved[r0:r1])[0]
        if mv.size:
            li = torch.as_tensor(mv, device=device)
            kk = torch.as_tensor(plan.peak[r0:r1][mv], device=device)
            jj = torch.as_tensor(plan.moved_to[r0:r1][mv], device=device)
            a = zq[li, kk].clone()
            b = zq[li, jj].clone()
            zq[li, kk] = b
            zq[li, jj] = a
        return zb, zq
    if cfg.kind == "student":
        z0 = _randn(shape, _block_seed(cfg, 0, blk), device)
        chi = torch.zeros(shape, device=device, dtype=torch.float32)
        for t in range(p["nu"]):
            chi += _randn(shape, _block_seed(cfg, 10 + t, blk), device).square()
        zb = (p["scale"] * z0 / torch.sqrt(chi / p["nu"])).to(bt)
        del chi, z0
        m = 1.0 + p["mult_sigma"] * _randn(shape, _block_seed(cfg, 1, blk), device)
        a = p["add_sigma"] * _randn(shape, _block_seed(cfg, 2, blk), device)
        zq = (zb.float() * m + a).to(qt)
        return zb, zq
    if cfg.kind == "ties":
        zb = (p["base_sigma"] * _randn(shape, _block_seed(cfg, 0, blk), device)).to(bt)
        third = torch.div(rows * 3, cfg.n_rows, rounding_mode="floor").clamp(max=2)
        sig = torch.tensor(p["sigmas"], device=device, dtype=torch.float32)[third]
        zq = (zb.float() + sig[:, None] * _randn(shape, _block_seed(cfg, 1, blk), device)).to(qt)
        tr = np.nonzero(plan.tie[r0:r1])[0]
        if tr.size:
            li = torch.as_tensor(tr, device=device)
            ii = torch.as_tensor(plan.tie_i[r0:r1][tr], device=device)
            jj = torch.as_tensor(plan.tie_j[r0:r1][tr], device=device)
            vb = (zb[li].float().max(dim=1).values + 1.0).to(bt)
            vq = (zq[li].float().max(dim=1).values + 1.0).to(qt)
            zb[li, ii] = vb
            zb[li, jj] = vb
            zq[li, ii] = vq
            zq[li, jj] = vq
        return zb, zq
    raise ValueError(f"unknown generator kind {cfg.kind}")


def fill(cfg: Config, base: torch.Tensor, quant: torch.Tensor, r0: int = 0,
         plan: RowPlan | None = None) -> None:
    """Write rows [r0, r0 + base.shape[0]) of the configuration into base/quant."""
    plan = plan or row_plan(cfg)
    n = base.shape[0]
    r = r0
    while r < r0 + n:
        b0 = (r // BLOCK_ROWS) * BLOCK_ROWS
        b1 = min(b0 + BLOCK_ROWS, cfg.n_rows)
        zb, zq = _fill_block(cfg, plan, b0, b1, base.device)
        lo, hi = r - b0, min(b1, r0 + n) - b0
        base[r - r0:r - r0 + hi - lo].copy_(zb[lo:hi])
        quant[r - r0:r - r0 + hi - lo].copy_(zq[lo:hi])
        r = b0 + hi
    return None


def generate(cfg: Config, r0: int = 0, r1: int | None = None, device="cpu"):
    """Allocate and fill rows [r0, r1) of a configuration on ``device``."""
    r1 = cfg.n_rows if r1 is None else r1
    base = torch.empty((r1 - r0, cfg.vocab), dtype=torch_dtype(cfg.base_dtype), device=device)
    quant = torch.empty((r1 - r0, cfg.vocab), dtype=torch_dtype(cfg.quant_dtype), device=device)
    fill(cfg, base, quant, r0)
    return base, quant


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy in the oracle's input convention (bf16 as raw uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# Token ids for the token-conditioned metrics. Each row stands for one position
# of a text, and its token id is the token that follows that position. The
# text is not available, so the ids are drawn: uniformly over the vocabulary,
# except that on configurations with a planted peak half of the rows take the
# peak's index (a confident model that is right about half the time). The last
# position of every context has no following token and gets -1 (not scored).
CONTEXT_ROWS = 8192


def tokens(cfg: Config, r0: int = 0, r1: int | None = None, plan: RowPlan | None = None) -> np.ndarray:
    """int32 token ids for rows [r0, r1) of a configuration (host array)."""
    r1 = cfg.n_rows if r1 is None else r1
    g = _rng(cfg, 7)
    ids = g.integers(0, cfg.vocab, size=cfg.n_rows).astype(np.int64)
    if cfg.kind == "peak":
        plan = plan or row_plan(cfg)
        use_peak = g.random(cfg.n_rows) < 0.5
        ids = np.where(use_peak, plan.peak, ids)
    last = (np.arange(cfg.n_rows) % CONTEXT_ROWS) == CONTEXT_ROWS - 1
    ids[last] = -1
    return ids[r0:r1].astype(np.int32)
