"""Seeded synthetic inputs shaped like the workloads of the page "DLRM For PyTorch".

The page trains on Criteo Terabyte (13 numerical + 26 categorical features, §Getting the
data / §Dataset guidelines) and offers a synthetic dataset of 26 tables x 100,000 rows
(§Command-line options, --synthetic_dataset_table_sizes).  None of those data are used
here: every buffer is drawn from seeded generators with the shapes and distributions of
the workloads listed in ``WORKLOADS``.

This module only draws random inputs; it holds none of the embedding / interaction
arithmetic.  The bottom MLP that turns the dense features into x0 is input preparation
(x0 is an input of the interaction), run with plain torch ops in fp32.

Recipe (all from base seed 12345, the page's --seed default):
  * tables: N(0, 0.01) per element (sigma = 0.01), in the table dtype;
  * indices: per table, uniform over its rows, or truncated Zipf(alpha) over ranks 1..n
    (P(k) ~ k^-alpha, exact inverse CDF) mapped to rows by a seeded affine bijection
    row = (a * (k - 1) + c) mod n with gcd(a, n) = 1, so hot rows are scattered; for
    measurement controls also "distinct": a seeded random permutation of the rows (no row
    looked up twice while the table has at least as many rows as lookups);
  * bag lengths: 1, or Poisson(mean) clipped to [lo, hi], independently per bag;
  * dense features: exp(N(0, 1)) (log-normal), 13 per sample;
  * x0: bottom MLP with ReLU after every layer, weights and biases U(+-1/sqrt(fan_in));
  * upstream gradient of the interaction output: N(0, 1), padding columns zero.
Each buffer has its own seed, derived from (base seed, buffer name, table, batch number).
"""
import dataclasses
import math
import zlib
from typing import List, Optional, Tuple

import numpy as np
import torch

BASE_SEED = 12345
_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def large_table_rows(num: int = 26, lo: int = 4, hi: int = 40_000_000, total: int = 200_000_000) -> List[int]:
    """Table sizes from `lo` to `hi` on a warped log grid n_i = round(lo * (hi/lo)^((i/(num-1))^g)),
    with g chosen by bisection so that the sizes add up to `total` rows (26 tables,
    4 .. 40,000,000 rows, ~200M rows in all)."""
    def sizes(g):
        return [int(round(lo * (hi / lo) ** ((i / (num - 1)) ** g))) for i in range(num)]
    a, b = 0.01, 1.0
    for _ in range(100):
        m = (a + b) / 2
        if sum(sizes(m)) > total:
            a = m
        else:
            b = m
    return sizes(a)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    rows: Tuple[int, ...]
    dim: int
    table_dtype: str
    act_dtype: str
    index_dist: str  # "uniform", "zipf" or "distinct" (rows without repeats, a measurement control)
    zipf_alpha: float = 0.0
    bag: Tuple = ("one",)  # ("one",) or ("poisson", mean, lo, hi)
    bottom_mlp: Tuple[int, ...] = (13, 512, 256, 128)
    backward: bool = True
    lr: float = 0.01
    description: str = ""

    @property
    def num_tables(self) -> int:
        return len(self.rows)

    @property
    def total_rows(self) -> int:
        return int(sum(self.rows))

    @property
    def num_pairs(self) -> int:
        v = self.num_tables + 1
        return v * (v - 1) // 2

    @property
    def out_width(self) -> int:
        return self.dim + self.num_pairs

    @property
    def out_stride(self) -> int:
        """Interaction output row padded with zeros to a multiple of 16 bytes."""
        per = 16 // torch.tensor([], dtype=_TORCH[self.act_dtype]).element_size()
        return (self.out_width + per - 1) // per * per

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 256, (1000,) * 8, 16, "f32", "f32", "uniform", bottom_mlp=(13, 64, 16),
        description="B=256, 8 tables x 1000 x 16 fp32, hotness 1 uniform, bottom MLP 13-64-16, "
                    "9 vectors -> 36 pairs -> 52 features, fwd+bwd+SGD lr 0.01"),
    "fwd_core": Workload(
        "fwd_core", 65536, (100_000,) * 26, 128, "f32", "bf16", "zipf", 1.05, backward=False,
        description="B=65536, 26 tables x 100000 x 128 fp32, bf16 activations, Zipf(1.05) hotness 1, "
                    "27 vectors -> 351 pairs -> 479 padded to 480"),
    "train_step": Workload(
        "train_step", 65536, (100_000,) * 26, 128, "f32", "bf16", "zipf", 1.05, backward=True,
        description="fwd_core shapes + interaction backward + sort/segment-reduce/SGD (lr 0.01) "
                    "on the fp32 tables"),
    "large_table": Workload(
        "large_table", 262144, tuple(large_table_rows()), 128, "f16", "f16", "zipf", 1.1, backward=False,
        description="B=262144, 26 fp16 tables of 4 .. 40M rows (200M rows, 51.2 GB), Zipf(1.1) "
                    "hotness 1, fp16 activations, forward only"),
    "multi_hot": Workload(
        "multi_hot", 16384, (1_000_000,) * 100, 64, "bf16", "bf16", "zipf", 1.05,
        bag=("poisson", 20.0, 1, 100), bottom_mlp=(13, 512, 256, 64), backward=True,
        description="B=16384, 100 bf16 tables x 1M x 64, bag length Poisson(20) clipped to [1,100], "
                    "Zipf(1.05), 101 vectors -> 5050 pairs, fwd+bwd+update"),
    # the multi-hot shapes forward only (serving: the fused forward, pooled vectors kept on chip)
    "multi_hot_infer": Workload(
        "multi_hot_infer", 16384, (1_000_000,) * 100, 64, "bf16", "bf16", "zipf", 1.05,
        bag=("poisson", 20.0, 1, 100), bottom_mlp=(13, 512, 256, 64), backward=False,
        description="multi_hot shapes, forward only (fused gather + interaction, pooled vectors "
                    "not stored)"),
    # secondary figure: the small tables at the large batch (cache-resident tables)
    "train_small_tables": Workload(
        "train_small_tables", 65536, (1000,) * 8, 16, "f32", "bf16", "zipf", 1.05,
        bottom_mlp=(13, 64, 16), backward=True,
        description="B=65536, 8 tables x 1000 x 16 fp32 (cache-resident), bf16 activations, "
                    "Zipf(1.05) hotness 1, 9 vectors -> 36 pairs -> 52 padded to 56, fwd+bwd+SGD"),
    # controls.  Uniform indices still repeat rows (65,536 lookups into a 100,000-row table
    # touch ~48,000 rows), and a table processed table-major fits in the memory-side cache,
    # so uniform lookups are partly served from cache; distinct rows are the honest test of
    # HBM bandwidth: every row is read once, from HBM
    "fwd_core_uniform": Workload(
        "fwd_core_uniform", 65536, (100_000,) * 26, 128, "f32", "bf16", "uniform", backward=False,
        description="fwd_core shapes with uniform indices (control: less row reuse)"),
    "fwd_core_distinct": Workload(
        "fwd_core_distinct", 65536, (100_000,) * 26, 128, "f32", "bf16", "distinct", backward=False,
        description="fwd_core shapes, each table's lookups distinct rows (control: no row reuse)"),
    "large_table_uniform": Workload(
        "large_table_uniform", 262144, tuple(large_table_rows()), 128, "f16", "f16", "uniform",
        backward=False,
        description="large_table shapes with uniform indices (control: row reuse only in the small "
                    "tables)"),
}


def seed_for(*tags) -> int:
    """A 63-bit seed for one buffer, from the base seed and the buffer's tags."""
    words = [BASE_SEED] + [zlib.crc32(str(t).encode()) for t in tags]
    return int(np.random.SeedSequence(words).generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def _gen(device, *tags) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*tags))
    return g


def make_tables(wl: Workload, device, chunk_rows: int = 1 << 22) -> Tuple[torch.Tensor, torch.Tensor]:
    """Joint table [total_rows, D] (table dtype) and row_offset int64 [F+1] on `device`."""
    W = torch.empty((wl.total_rows, wl.dim), dtype=_TORCH[wl.table_dtype], device=device)
    g = _gen(device, wl.name, "tables")
    for r0 in range(0, wl.total_rows, chunk_rows):
        r1 = min(r0 + chunk_rows, wl.total_rows)
        x = torch.randn((r1 - r0, wl.dim), generator=g, device=device, dtype=torch.float32)
        W[r0:r1] = (x * 0.01).to(W.dtype)
    row_offset = torch.tensor(np.concatenate([[0], np.cumsum(wl.rows)]), dtype=torch.int64, device=device)
    return W, row_offset


_CDF_CACHE = {}


def _zipf_cdf(n: int, alpha: float, device) -> torch.Tensor:
    key = (n, alpha, str(device))
    if key not in _CDF_CACHE:
        k = torch.arange(1, n + 1, dtype=torch.float64, device=device)
        c = torch.cumsum(k.pow(-alpha), 0)
        _CDF_CACHE[key] = c / c[-1]
    return _CDF_CACHE[key]


def _affine(n: int, rng: np.random.Generator) -> Tuple[int, int]:
    if n == 1:
        return 1, 0
    while True:
        a = int(rng.integers(1, n))
        if math.gcd(a, n) == 1:
            return a, int(rng.integers(0, n))


def bag_lengths(wl: Workload, device, batch_id: int = 0) -> torch.Tensor:
    """int64 [F, B] bag lengths."""
    F, B = wl.num_tables, wl.batch
    if wl.bag[0] == "one":
        return torch.ones((F, B), dtype=torch.int64, device=device)
    _, mean, lo, hi = wl.bag
    g = _gen(device, wl.name, "bag_len", batch_id)
    lam = torch.full((F, B), float(mean), dtype=torch.float32, device=device)
    return torch.poisson(lam, generator=g).to(torch.int64).clamp_(lo, hi)


def make_indices(wl: Workload, device, batch_id: int = 0):
    """(indices int32 [nnz], offsets int32 [F*B+1]) table-major CSR on `device`."""
    lens = bag_lengths(wl, device, batch_id)
    offsets = torch.zeros(lens.numel() + 1, dtype=torch.int64, device=device)
    offsets[1:] = torch.cumsum(lens.reshape(-1), 0)
    per_table = lens.sum(dim=1).tolist()
    parts = []
    for t, (n, m) in enumerate(zip(wl.rows, per_table)):
        g = _gen(device, wl.name, "indices", t, batch_id)
        if wl.index_dist == "uniform":
            parts.append(torch.randint(0, n, (m,), generator=g, device=device, dtype=torch.int64))
            continue
        if wl.index_dist == "distinct":
            # a seeded random permutation of the table's rows, repeated only if the table has
            # fewer rows than lookups: no row is read twice, so no cache can serve a lookup
            reps = (m + n - 1) // n
            perm = torch.cat([torch.randperm(n, generator=g, device=device) for _ in range(max(reps, 1))])
            parts.append(perm[:m].to(torch.int64))
            continue
        u = torch.rand((m,), generator=g, device=device, dtype=torch.float64)
        rank = torch.searchsorted(_zipf_cdf(n, wl.zipf_alpha, device), u).clamp_(max=n - 1)  # rank - 1
        a, c = _affine(n, np.random.default_rng(seed_for(wl.name, "scatter", t)))
        parts.append((rank * a + c) % n)
    indices = torch.cat(parts).to(torch.int32) if parts else torch.zeros(0, dtype=torch.int32, device=device)
    return indices, offsets.to(torch.int32)


def make_x0(wl: Workload, device, batch_id: int = 0) -> torch.Tensor:
    """Bottom-MLP output [B, D] in the activation dtype (fp32 arithmetic)."""
    g = _gen(device, wl.name, "dense", batch_id)
    h = torch.exp(torch.randn((wl.batch, wl.bottom_mlp[0]), generator=g, device=device))
    gw = _gen(device, wl.name, "bottom_mlp")
    for fan_in, fan_out in zip(wl.bottom_mlp[:-1], wl.bottom_mlp[1:]):
        bound = 1.0 / math.sqrt(fan_in)
        w = (torch.rand((fan_in, fan_out), generator=gw, device=device) * 2 - 1) * bound
        b = (torch.rand((fan_out,), generator=gw, device=device) * 2 - 1) * bound
        h = torch.relu(h @ w + b)
    return h.to(_TORCH[wl.act_dtype]).contiguous()


def make_dout(wl: Workload, device, batch_id: int = 0) -> torch.Tensor:
    """Upstream gradient [B, out_stride] of the interaction output, N(0,1), zero padding."""
    g = _gen(device, wl.name, "dout", batch_id)
    G = torch.randn((wl.batch, wl.out_stride), generator=g, device=device)
    G[:, wl.out_width:] = 0
    return G.to(_TORCH[wl.act_dtype]).contiguous()


TOP_MLP = (1024, 1024, 512, 256, 1)  # --top_mlp_sizes default
LABEL_RATE = 0.25  # clicks per sample of the synthetic labels (the page gives no rate)


def make_dense(wl: Workload, device, batch_id: int = 0, k_pad: int = 16) -> torch.Tensor:
    """The dense features of make_x0 (exp(N(0,1)), 13 per sample) in the activation dtype,
    zero-padded to k_pad columns so that rows are 16-byte multiples."""
    g = _gen(device, wl.name, "dense", batch_id)
    h = torch.exp(torch.randn((wl.batch, wl.bottom_mlp[0]), generator=g, device=device))
    out = torch.zeros((wl.batch, k_pad), dtype=_TORCH[wl.act_dtype], device=device)
    out[:, :wl.bottom_mlp[0]] = h.to(out.dtype)
    return out


def make_mlp_params(wl: Workload, which: str, sizes, k_pad: int, device):
    """Dense-layer parameters [(w [N][K'] fp32, b [N] fp32)], w and b ~ U(+-1/sqrt(fan_in));
    the first layer's input width is zero-padded from sizes[0] to k_pad columns."""
    gw = _gen(device, wl.name, which + "_mlp")
    params = []
    for i, (fan_in, fan_out) in enumerate(zip(sizes[:-1], sizes[1:])):
        bound = 1.0 / math.sqrt(fan_in)
        k = k_pad if i == 0 else fan_in
        w = torch.zeros((fan_out, k), dtype=torch.float32, device=device)
        w[:, :fan_in] = (torch.rand((fan_out, fan_in), generator=gw, device=device) * 2 - 1) * bound
        b = (torch.rand((fan_out,), generator=gw, device=device) * 2 - 1) * bound
        params.append((w, b))
    return params


def make_labels(wl: Workload, device, batch_id: int = 0, rate: float = LABEL_RATE) -> torch.Tensor:
    """Click labels in {0, 1} (fp32 [B]), Bernoulli(rate)."""
    g = _gen(device, wl.name, "labels", batch_id)
    return (torch.rand((wl.batch,), generator=g, device=device) < rate).to(torch.float32)


def make_normal(shape, device, dtype: str, *tags, scale: float = 1.0, relu: bool = False) -> torch.Tensor:
    """A seeded N(0, scale^2) tensor (optionally passed through max(., 0)) in `dtype`, for
    testing a call on its own."""
    x = torch.randn(shape, generator=_gen(device, *tags), device=device) * scale
    if relu:
        x = torch.clamp_min(x, 0.0)
    return x.to(_TORCH[dtype]).contiguous()


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH[name]


def act_dtype(wl: Workload) -> torch.dtype:
    return _TORCH[wl.act_dtype]


def table_dtype(wl: Workload) -> torch.dtype:
    return _TORCH[wl.table_dtype]


def make_emb(wl: Workload, device, batch_id: int = 0, sigma: float = 0.02) -> torch.Tensor:
    """Stand-in pooled embeddings [B, F, D] (N(0, sigma)) in the activation dtype, for
    testing the interaction on its own."""
    g = _gen(device, wl.name, "emb", batch_id)
    x = torch.randn((wl.batch, wl.num_tables, wl.dim), generator=g, device=device) * sigma
    return x.to(_TORCH[wl.act_dtype]).contiguous()


def make_demb(wl: Workload, device, batch_id: int = 0, dtype: Optional[str] = None) -> torch.Tensor:
    """Stand-in embedding gradients [B, F, D] (N(0, 1)), for testing the update on its own."""
    g = _gen(device, wl.name, "demb", batch_id)
    x = torch.randn((wl.batch, wl.num_tables, wl.dim), generator=g, device=device)
    return x.to(_TORCH[dtype or wl.act_dtype]).contiguous()
