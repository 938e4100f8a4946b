"""Seeded synthetic inputs for the DLRMv1 forward hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, no dot products, no layers), so that both the
CPU oracle's tests and the HIP path can take their inputs from it.

Recipe (every stream is seeded from a base seed and a fixed stream number):
  table k        stream 1000 + k   N(0, std^2) float32, std = 0.01
  indices of k   stream 2000 + k   int32, uniform on [0, rows) or bounded Zipf
  dense input    stream 3000       N(0, 1) float32
  MLP layer i    stream 4000 + i   Xavier-uniform weight, zero bias
  weights of k   stream 5000 + k   per-sample weights, U[0, 1) float32
  lengths of k   stream 6000 + k   CSR bag sizes, uniform integers on [0, 2L]
bfloat16 tables keep the high 16 bits of the float32 draw (truncation), as
bit patterns (uint16 on the host, torch.bfloat16 on the device).  FP8 E4M3
tables hold the draw divided by FP8_SCALE = 2^-8, rounded to the nearest
E4M3 value by torch's float8_e4m3fn conversion (uint8 codes on the host,
torch.float8_e4m3fn on the device), and are pooled with that scale.
CSR workloads draw one bag size per (sample, table), mean L, empty bags
included; the indices of table k then number the sum of its sizes and the
offsets are the exclusive prefix sums of the sizes.
Bounded Zipf(s) draws rank r in 1..N with probability proportional to r^-s
by inverse CDF, then scatters ranks over rows with the bijection
row = (a (r - 1) + 7919 k) mod N, a = 999983 (prime), so hot rows are not
adjacent in memory.  Offsets are uniform stride: arange(0, B*L, L).

Small tables are drawn on the host with numpy (PCG64); tables too large for
that are drawn on the device with torch's CUDA generator (see
`table_device`).  Both are plain N(0, std^2) samples; which one a workload
uses is recorded in `Workload.table_source`.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field

import numpy as np

ZIPF_SCATTER_MUL = 999_983
ZIPF_SCATTER_ADD = 7_919


@dataclass(frozen=True)
class Workload:
    """Shape and value distribution of one forward batch."""
    name: str
    batch: int
    num_tables: int
    rows: int
    dim: int
    bag: int
    dist: str                      # "uniform" or "zipf"
    zipf_s: float = 1.05
    table_std: float = 0.01
    dense_in: int = 0              # 0: dense (B, dim) is given directly
    bottom: tuple = ()             # bottom MLP widths after dense_in
    top: tuple = ()                # top MLP widths after the interaction
    table_source: str = "host"     # "host" (numpy) or "device" (torch CUDA)
    table_dtype: str = "f32"       # "f32", "bf16" or "fp8" (E4M3) table storage
    pool: str = "sum"              # "sum" or "mean"
    weighted: bool = False         # per-sample weights (sum only)
    lengths: str = "fixed"         # "fixed" (L per bag) or "uniform" (0..2L, CSR)
    description: str = field(default="", compare=False)

    @property
    def num_features(self) -> int:
        return self.num_tables + 1

    @property
    def num_pairs(self) -> int:
        f = self.num_features
        return f * (f - 1) // 2

    @property
    def out_width(self) -> int:
        return self.dim + self.num_pairs


WORKLOADS = {
    "tiny": Workload(
        "tiny", batch=32, num_tables=2, rows=1000, dim=16, bag=4, dist="uniform",
        description="B=32, K=2 tables x 1000 rows x D=16, 4 indices/bag uniform"),
    "mid": Workload(
        "mid", batch=2048, num_tables=8, rows=100_000, dim=64, bag=20,
        dist="uniform",
        description="B=2048, K=8 tables x 100,000 rows x D=64, 20 indices/bag "
                    "uniform"),
    "nc32": Workload(
        "nc32", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="zipf", table_source="device",
        description="B=2048, K=32 tables x 1,000,000 rows x D=64, 20 indices/bag "
                    "Zipf(1.05)"),
    "nc32-uniform": Workload(
        "nc32-uniform", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="uniform", table_source="device",
        description="nc32 with uniform indices (no hot rows)"),
    "large": Workload(
        "large", batch=16384, num_tables=26, rows=4_000_000, dim=128, bag=40,
        dist="zipf", table_source="device",
        description="B=16384, K=26 tables x 4,000,000 rows x D=128 (~53 GB), "
                    "40 indices/bag Zipf(1.05)"),
    "large-uniform": Workload(
        "large-uniform", batch=16384, num_tables=26, rows=4_000_000, dim=128, bag=40,
        dist="uniform", table_source="device",
        description="large with uniform indices (no hot rows)"),
    "nc32-bf16": Workload(
        "nc32-bf16", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="zipf", table_source="device", table_dtype="bf16",
        description="nc32 with bfloat16 tables (128-byte rows)"),
    "nc32-fp8": Workload(
        "nc32-fp8", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="zipf", table_source="device", table_dtype="fp8",
        description="nc32 with FP8 E4M3 tables (64-byte rows, scale 2^-8)"),
    "nc32-mean": Workload(
        "nc32-mean", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="zipf", table_source="device", pool="mean",
        description="nc32 with mean pooling"),
    "nc32-weighted": Workload(
        "nc32-weighted", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="zipf", table_source="device", weighted=True,
        description="nc32 with per-sample weights U[0, 1)"),
    "nc32-csr": Workload(
        "nc32-csr", batch=2048, num_tables=32, rows=1_000_000, dim=64, bag=20,
        dist="zipf", table_source="device", lengths="uniform",
        description="nc32 with CSR bags of uniform size on [0, 40] (mean 20)"),
    "dlrm": Workload(
        "dlrm", batch=8192, num_tables=26, rows=1_000_000, dim=64, bag=20,
        dist="zipf", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1),
        table_source="device",
        description="DLRMv1 forward: dense 13 -> 512-256-64, K=26 tables x "
                    "1,000,000 rows x D=64, 20 indices/bag Zipf(1.05), top "
                    "415 -> 512-256-1"),
}


def cell_workload(num_tables: int, batch: int) -> Workload:
    """The pages' small DLRMv1 cell: 3 dense features, D=16, 2 indices per bag
    uniform over 4096-row tables; bottom MLP 3-16 and top MLP (16+P)-16-1
    (the pages do not print the MLP widths)."""
    return Workload(f"cell-nc{num_tables}-b{batch}", batch=batch, num_tables=num_tables,
                    rows=4096, dim=16, bag=2, dist="uniform", dense_in=3, bottom=(16,),
                    top=(16, 1),
                    description=f"pages' cell: nc={num_tables}, b={batch}, 3 dense, D=16, "
                                f"L=2, 4096 rows, MLPs 3-16 and (16+P)-16-1")


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream)]))


def torch_seed(seed: int, stream: int) -> int:
    """Integer seed for torch's generator for (base seed, stream)."""
    return int(seed) * 1_000_003 + int(stream)


@functools.lru_cache(maxsize=8)
def _zipf_cdf(n: int, s: float) -> np.ndarray:
    weights = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return np.cumsum(weights)


def zipf_ranks(rng: np.random.Generator, n: int, s: float, count: int) -> np.ndarray:
    """0-based ranks drawn from a bounded Zipf(s) over n ranks (inverse CDF)."""
    cdf = _zipf_cdf(n, s)
    u = rng.random(count) * cdf[-1]
    r = np.searchsorted(cdf, u, side="right")
    return np.minimum(r, n - 1)


def scatter_ranks(ranks: np.ndarray, n: int, table: int) -> np.ndarray:
    """Bijection from ranks to rows: (a r + 7919 k) mod n."""
    a = ZIPF_SCATTER_MUL
    while math.gcd(a, n) != 1:
        a += 2
    return (ranks.astype(np.int64) * a + ZIPF_SCATTER_ADD * table) % n


def bag_lengths(w: Workload, table: int, seed: int = 0, batch: int = None) -> np.ndarray:
    """(B,) int64 bag sizes of table `table`: L each, or uniform on [0, 2L]."""
    b = w.batch if batch is None else batch
    if w.lengths == "fixed":
        return np.full(b, w.bag, np.int64)
    if w.lengths == "uniform":
        return _rng(seed, 6000 + table).integers(0, 2 * w.bag + 1, size=b, dtype=np.int64)
    raise ValueError(f"unknown bag-length mix {w.lengths!r}")


def csr_offsets(w: Workload, table: int, seed: int = 0, batch: int = None) -> np.ndarray:
    """(B,) int32 bag starts: exclusive prefix sums of bag_lengths."""
    lens = bag_lengths(w, table, seed, batch)
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)


def indices(w: Workload, table: int, seed: int = 0, batch: int = None) -> np.ndarray:
    """(n_idx,) int32 row indices of table `table` (n_idx = B*L for fixed bags)."""
    b = w.batch if batch is None else batch
    count = int(bag_lengths(w, table, seed, b).sum())
    rng = _rng(seed, 2000 + table)
    if w.dist == "uniform":
        idx = rng.integers(0, w.rows, size=count, dtype=np.int64)
    elif w.dist == "zipf":
        idx = scatter_ranks(zipf_ranks(rng, w.rows, w.zipf_s, count), w.rows, table)
    else:
        raise ValueError(f"unknown index distribution {w.dist!r}")
    return idx.astype(np.int32)


def offsets(w: Workload, batch: int = None) -> np.ndarray:
    """Uniform-stride bag starts arange(0, B*L, L) as (B,) int32."""
    b = w.batch if batch is None else batch
    return np.arange(0, b * w.bag, w.bag, dtype=np.int32)


def dense(w: Workload, seed: int = 0, batch: int = None) -> np.ndarray:
    """(B, dense width) float32 N(0, 1); the width is dense_in or dim."""
    b = w.batch if batch is None else batch
    width = w.dense_in if w.dense_in else w.dim
    return _rng(seed, 3000).standard_normal((b, width), dtype=np.float32)


def table_host(w: Workload, table: int, seed: int = 0, rows: int = None) -> np.ndarray:
    """(rows, D) float32 N(0, std^2) drawn with numpy."""
    r = w.rows if rows is None else rows
    x = _rng(seed, 1000 + table).standard_normal((r, w.dim), dtype=np.float32)
    x *= np.float32(w.table_std)
    return x


def table_device(w: Workload, table: int, seed: int = 0, device="cuda", rows: int = None):
    """(rows, D) float32 N(0, std^2) drawn on the device with torch."""
    import torch
    r = w.rows if rows is None else rows
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, 1000 + table))
    t = torch.randn((r, w.dim), generator=g, device=device, dtype=torch.float32)
    return t.mul_(w.table_std)


def sample_weights(w: Workload, table: int, n: int, seed: int = 0) -> np.ndarray:
    """(n,) float32 per-sample weights U[0, 1) of table `table`."""
    return _rng(seed, 5000 + table).random(n, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) holding the high half of float32 x."""
    x = np.ascontiguousarray(x, np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


FP8_SCALE = 2.0 ** -8


def table_scale(w: Workload):
    """Per-table scale of the workload's storage (None: no scaling)."""
    return FP8_SCALE if w.table_dtype == "fp8" else None


def fp8_codes(x: np.ndarray) -> np.ndarray:
    """uint8 FP8 E4M3 codes of x / FP8_SCALE (torch's float8_e4m3fn rounding)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32) / np.float32(FP8_SCALE))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def table_host_typed(w: Workload, table: int, seed: int = 0, rows: int = None) -> np.ndarray:
    """table_host in the workload's storage type (uint16 bit patterns for bf16,
    uint8 codes for fp8)."""
    t = table_host(w, table, seed, rows)
    if w.table_dtype == "bf16":
        return bf16_bits(t)
    if w.table_dtype == "fp8":
        return fp8_codes(t)
    return t


def table_device_typed(w: Workload, table: int, seed: int = 0, device="cuda",
                       rows: int = None):
    """table_device in the workload's storage type (torch.bfloat16 for bf16)."""
    import torch
    t = table_device(w, table, seed, device, rows)
    if w.table_dtype == "fp8":
        return t.div_(FP8_SCALE).to(torch.float8_e4m3fn)
    if w.table_dtype != "bf16":
        return t
    return (t.view(torch.int32) >> 16).to(torch.int16).view(torch.bfloat16)


def dyadic(rng: np.random.Generator, shape, scale_bits: int = 8,
           max_int: int = 128) -> np.ndarray:
    """Values n / 2^scale_bits with n uniform in [-max_int, max_int), float32.

    While every partial sum, in units of the smallest product, stays below
    2^24, sums and products of such values are exact in float32, so every
    summation order gives the same bits (see dyadic_max_int).
    """
    n = rng.integers(-max_int, max_int, size=shape, dtype=np.int64)
    return (n.astype(np.float32) / np.float32(2 ** scale_bits)).astype(np.float32)


def dyadic_max_int(dim: int, bag: int) -> int:
    """Largest power-of-two integer range keeping pooled dot products exact.

    A bag sum is at most bag * max_int units and a dot of two of them at most
    dim * bag^2 * max_int^2 units squared; that must stay below 2^24.
    """
    m = 128
    while m > 1 and dim * max(bag, 1) ** 2 * m * m >= 2 ** 24:
        m //= 2
    return m


def table_dyadic(w: Workload, table: int, seed: int = 0, rows: int = None) -> np.ndarray:
    r = w.rows if rows is None else rows
    return dyadic(_rng(seed, 1000 + table), (r, w.dim), max_int=dyadic_max_int(w.dim, w.bag))


def dense_dyadic(w: Workload, seed: int = 0, batch: int = None) -> np.ndarray:
    b = w.batch if batch is None else batch
    return dyadic(_rng(seed, 3000), (b, w.dense_in if w.dense_in else w.dim),
                  max_int=dyadic_max_int(w.dim, w.bag))


def mlp(widths, seed: int = 0, first_stream: int = 4000, bias_std: float = 0.0):
    """Xavier-uniform weights (out, in) float32 and biases for a layer stack.

    widths = (in, h1, h2, ..., out).  Bias is zero unless bias_std > 0.
    """
    layers = []
    for i in range(len(widths) - 1):
        fan_in, fan_out = widths[i], widths[i + 1]
        rng = _rng(seed, first_stream + i)
        bound = math.sqrt(6.0 / (fan_in + fan_out))
        wgt = rng.uniform(-bound, bound, size=(fan_out, fan_in)).astype(np.float32)
        if bias_std > 0:
            b = (rng.standard_normal(fan_out) * bias_std).astype(np.float32)
        else:
            b = np.zeros(fan_out, np.float32)
        layers.append((wgt, b))
    return layers


def dlrm_layers(w: Workload, seed: int = 0, bias_std: float = 0.0):
    """(bottom, top) lists of (weight, bias, act) for a full-forward workload."""
    bw = (w.dense_in,) + tuple(w.bottom)
    tw = (w.out_width,) + tuple(w.top)
    bottom = [(wt, b, "relu") for wt, b in mlp(bw, seed, 4000, bias_std)]
    top_l = mlp(tw, seed, 4100, bias_std)
    top = [(wt, b, "relu" if i + 1 < len(top_l) else "sigmoid")
           for i, (wt, b) in enumerate(top_l)]
    return bottom, top
