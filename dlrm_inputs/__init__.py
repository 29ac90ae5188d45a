"""Seeded synthetic inputs for the DLRMv1 forward hot path.

This module is shared by the HIP path, the fp64 oracle and the benchmark. It
holds workload shapes and random-number draws only: none of the method's
arithmetic (no gathers, dots, matmuls or activations) lives here.

Workloads (all fp32 values, int64 indices/offsets, synthetic):

* ``tiny``       batch 8, 4 dense, 3 tables x 1000 rows x d=16, bag 1,
                 bottom 4-32-16, top 22-32-1, zero biases.
* ``page4``      batch 2048, 13 dense, 3 tables x 100000 x d=64, bag 1,
                 bottom 13-512-256-64, top 70-512-256-1.
* ``manytable``  as ``page4`` with 32 tables, top 592-512-256-1.
* ``sweep``      batch in {16..16384} x tables in {1,4,8,16,32}, as ``page4``
                 otherwise, top (64+P)-512-256-1.
* ``stress``     batch 65536, 26 tables x 1e6 rows x d=128 (13.3 GB), fixed
                 bag 20, Zipf(1.05) indices, bottom 13-512-256-128,
                 top 479-1024-1024-512-256-1.

Distributions: dense ~ U[0,1); tables ~ N(0, 1/D); Linear weights
~ N(0, 1/fan_in) (the second parameter is a variance); biases zero for
``tiny`` and ~ N(0, 1/fan_in) elsewhere; indices uniform over rows, or a
bounded Zipf law P(row=k) proportional to (k+1)^-s over k in [0, V) drawn by
inverse CDF; offsets = L * arange(batch) (every bag holds L indices).

Seeding: tensor number k of workload number c is drawn from a generator seeded
``BASE_SEED + 1000*c + k``; k enumerates dense, tables, indices, bottom
weight/bias pairs, top weight/bias pairs, in that order.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

BASE_SEED = 20261202

SWEEP_BATCHES = (16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384)
SWEEP_TABLES = (1, 4, 8, 16, 32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    n_dense: int
    num_tables: int
    rows: int
    dim: int
    bag: int
    dist: str            # "uniform" or "zipf"
    ln_bot: tuple
    ln_top: tuple
    zero_bias: bool = False
    zipf_s: float = 1.05

    @property
    def n_feat(self) -> int:
        return self.num_tables + 1

    @property
    def n_pairs(self) -> int:
        f = self.n_feat
        return f * (f - 1) // 2

    def with_batch(self, batch: int) -> "Workload":
        return dataclasses.replace(self, batch=batch)


def _top(dim: int, tables: int, hidden=(512, 256)) -> tuple:
    f = tables + 1
    return (dim + f * (f - 1) // 2,) + tuple(hidden) + (1,)


TINY = Workload("tiny", 1, 8, 4, 3, 1000, 16, 1, "uniform", (4, 32, 16), (22, 32, 1), zero_bias=True)
PAGE4 = Workload("page4", 2, 2048, 13, 3, 100_000, 64, 1, "uniform", (13, 512, 256, 64), (70, 512, 256, 1))
MANYTABLE = Workload("manytable", 3, 2048, 13, 32, 100_000, 64, 1, "uniform", (13, 512, 256, 64), (592, 512, 256, 1))
STRESS = Workload("stress", 5, 65536, 13, 26, 1_000_000, 128, 20, "zipf", (13, 512, 256, 128),
                  (479, 1024, 1024, 512, 256, 1))


def sweep(batch: int, tables: int) -> Workload:
    """One cell of the batch x tables sweep grid (workload number 4)."""
    return Workload(f"sweep_b{batch}_t{tables}", 4, batch, 13, tables, 100_000, 64, 1, "uniform",
                    (13, 512, 256, 64), _top(64, tables))


WORKLOADS = {w.name: w for w in (TINY, PAGE4, MANYTABLE, STRESS)}


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name.startswith("sweep_b"):
        b, t = name[len("sweep_b"):].split("_t")
        return sweep(int(b), int(t))
    raise KeyError(name)


def custom(name: str, batch: int, n_dense: int, num_tables: int, rows: int, dim: int, bag: int,
           ln_bot, hidden_top=(32,), dist: str = "uniform", zero_bias: bool = False,
           cfg_id: int = 9) -> Workload:
    """A small workload with the same structure, for tests."""
    ln_bot = tuple(ln_bot)
    assert ln_bot[-1] == dim
    return Workload(name, cfg_id, batch, n_dense, num_tables, rows, dim, bag, dist, ln_bot,
                    _top(dim, num_tables, hidden_top), zero_bias=zero_bias)


@dataclasses.dataclass
class Inputs:
    """Everything one forward pass reads. Tensors live on one device."""
    workload: Workload
    dense: torch.Tensor                 # (B, n_dense) f32
    tables: List[torch.Tensor]          # T x (V, D) f32
    indices: List[torch.Tensor]         # T x (N_t,) int64
    offsets: List[torch.Tensor]         # T x (B,) int64, bag b = [off[b], off[b+1]) (last ends at N_t)
    bot_w: List[torch.Tensor]           # (out, in) f32
    bot_b: List[torch.Tensor]           # (out,) f32
    top_w: List[torch.Tensor]
    top_b: List[torch.Tensor]

    def to(self, device) -> "Inputs":
        mv = lambda xs: [x.to(device) for x in xs]
        return Inputs(self.workload, self.dense.to(device), mv(self.tables), mv(self.indices),
                      mv(self.offsets), mv(self.bot_w), mv(self.bot_b), mv(self.top_w), mv(self.top_b))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def zipf_cdf(rows: int, s: float, device="cpu") -> torch.Tensor:
    """Cumulative distribution of the bounded Zipf law over ranks 0..rows-1 (fp64)."""
    k = torch.arange(1, rows + 1, dtype=torch.float64, device=device)
    w = k.pow(-s)
    c = torch.cumsum(w, 0)
    return c / c[-1]


def draw_indices(n: int, rows: int, dist: str, gen: torch.Generator, device, zipf_s: float = 1.05,
                 cdf: Optional[torch.Tensor] = None) -> torch.Tensor:
    if dist == "uniform":
        return torch.randint(0, rows, (n,), generator=gen, device=device, dtype=torch.int64)
    if dist == "zipf":
        if cdf is None:
            cdf = zipf_cdf(rows, zipf_s, device)
        u = torch.rand(n, generator=gen, device=device, dtype=torch.float64)
        idx = torch.searchsorted(cdf, u, right=True)
        return idx.clamp_(max=rows - 1).to(torch.int64)
    raise ValueError(dist)


def make_inputs(w: Workload, device="cpu", int_tables: bool = False, int_dense: bool = False,
                seed: int = BASE_SEED) -> Inputs:
    """Draw every tensor of workload ``w`` on ``device``.

    ``int_tables`` swaps the N(0, 1/D) tables for integers in [-8, 8] stored as
    fp32, so that every bag sum is exact in fp32 whatever the summation order.
    ``int_dense`` does the same for the dense features with integers in [0, 4].
    """
    device = torch.device(device)
    base = seed + 1000 * w.cfg_id
    k = 0

    def nxt():
        nonlocal k
        g = _gen(device, base + k)
        k += 1
        return g

    B, D, T, V = w.batch, w.dim, w.num_tables, w.rows
    g = nxt()
    if int_dense:
        dense = torch.randint(0, 5, (B, w.n_dense), generator=g, device=device).to(torch.float32)
    else:
        dense = torch.rand((B, w.n_dense), generator=g, device=device, dtype=torch.float32)
    tables = []
    for _ in range(T):
        g = nxt()
        if int_tables:
            tables.append(torch.randint(-8, 9, (V, D), generator=g, device=device).to(torch.float32))
        else:
            t = torch.randn((V, D), generator=g, device=device, dtype=torch.float32)
            t.mul_(float(D) ** -0.5)
            tables.append(t)
    cdf = zipf_cdf(V, w.zipf_s, device) if w.dist == "zipf" else None
    indices, offsets = [], []
    for _ in range(T):
        g = nxt()
        indices.append(draw_indices(B * w.bag, V, w.dist, g, device, w.zipf_s, cdf))
        offsets.append(torch.arange(B, device=device, dtype=torch.int64) * w.bag)
    del cdf

    def linears(ln):
        ws, bs = [], []
        for i in range(len(ln) - 1):
            fan_in, fan_out = ln[i], ln[i + 1]
            g = nxt()
            W = torch.randn((fan_out, fan_in), generator=g, device=device, dtype=torch.float32)
            W.mul_(float(fan_in) ** -0.5)
            g = nxt()
            if w.zero_bias:
                b = torch.zeros((fan_out,), device=device, dtype=torch.float32)
            else:
                b = torch.randn((fan_out,), generator=g, device=device, dtype=torch.float32)
                b.mul_(float(fan_in) ** -0.5)
            ws.append(W)
            bs.append(b)
        return ws, bs

    bot_w, bot_b = linears(w.ln_bot)
    top_w, top_b = linears(w.ln_top)
    return Inputs(w, dense, tables, indices, offsets, bot_w, bot_b, top_w, top_b)


def make_indices(w: Workload, device="cpu", seed: int = BASE_SEED) -> List[torch.Tensor]:
    """Another independently drawn index set (T x (B*L,)) for workload ``w``."""
    device = torch.device(device)
    cdf = zipf_cdf(w.rows, w.zipf_s, device) if w.dist == "zipf" else None
    out = []
    for t in range(w.num_tables):
        g = _gen(device, seed + 1000 * w.cfg_id + 500 + t)
        out.append(draw_indices(w.batch * w.bag, w.rows, w.dist, g, device, w.zipf_s, cdf))
    return out


def ragged_bags(batch: int, max_len: int, gen_seed: int, empty_frac: float = 0.25):
    """Offsets (B,) int64 of bags with random lengths in [0, max_len], some empty.

    Returns ``(offsets, n_total)``; bag b spans [off[b], off[b+1]) and the last
    bag ends at ``n_total``.
    """
    g = _gen("cpu", gen_seed)
    lens = torch.randint(0, max_len + 1, (batch,), generator=g)
    lens[torch.rand(batch, generator=g) < empty_frac] = 0
    offs = torch.zeros(batch, dtype=torch.int64)
    if batch > 1:
        offs[1:] = torch.cumsum(lens[:-1], 0)
    return offs, int(lens.sum())


def subset(inp: Inputs, rows: torch.Tensor, compact_tables: bool = False) -> Inputs:
    """Inputs restricted to the samples ``rows`` (a 1-D index tensor), on the CPU.

    Each selected bag keeps its own indices; offsets are rebuilt for the
    packed index lists.  With ``compact_tables`` every table is replaced by
    just the rows the selected bags reference (indices renumbered to match),
    so a large resident table need not be copied whole.  Pure data
    selection, used to check sampled outputs of a large batch.
    """
    rows = rows.to("cpu")
    new_idx, new_off, new_tab = [], [], []
    for tab, idx, off in zip(inp.tables, inp.indices, inp.offsets):
        off_c = off.to("cpu")
        idx_c = idx.to("cpu")
        n = idx_c.numel()
        ends = torch.cat([off_c[1:], torch.tensor([n], dtype=torch.int64)])
        s, e = off_c[rows], ends[rows]
        lens = e - s
        # positions of every selected bag's indices, bag after bag, each bag's in order
        total = int(lens.sum())
        starts = torch.cumsum(lens, 0) - lens
        take = (torch.repeat_interleave(s, lens) +
                torch.arange(total, dtype=torch.int64) - torch.repeat_interleave(starts, lens))
        sel = idx_c[take]
        if compact_tables:
            uniq, inv = torch.unique(sel, return_inverse=True)
            if uniq.numel() == 0:
                uniq = torch.zeros(1, dtype=torch.int64)
            new_tab.append(tab[uniq.to(tab.device)].to("cpu"))
            new_idx.append(inv.to(torch.int64))
        else:
            new_tab.append(tab.to("cpu"))
            new_idx.append(sel)
        new_off.append(starts)
    w = inp.workload.with_batch(int(rows.numel()))
    cpu = lambda xs: [x.to("cpu") for x in xs]
    return Inputs(w, inp.dense.to("cpu")[rows], new_tab, new_idx, new_off,
                  cpu(inp.bot_w), cpu(inp.bot_b), cpu(inp.top_w), cpu(inp.top_b))
