"""Seeded synthetic inputs for the pooled-embedding path.

This module only *draws* inputs: table sizes, bag lengths, keys, upstream
gradients, and lays the keys out as table-major CSR. It holds none of the
arithmetic of the method (no pooling, dedup, reduction or optimizer step), so
both the HIP path and the CPU oracle may be fed from it.

Workload shapes follow the five configurations of the pooled-lookup benchmark:

  1  tiny: 4 fp32 tables, rows 1e3/5e3/1e4/5e4, dim 16, batch 128,
     bag length uniform in 1..4, uniform keys, sum pooling, SGD lr 0.01
  2  26 fp32 tables, rows log-uniform in [1e2, 1e6], dim 64, batch 16384,
     one-hot, Zipf(1.1) keys, sum pooling, Adagrad lr 0.01 eps 1e-8
  3  26 fp32 tables of 4M rows, dim 128, batch 65536, one-hot, Zipf(1.05),
     sum pooling, Adagrad (fp32 state)
  4  100 bf16 tables of 1M rows, dim 128, batch 32768, per-table hotness
     log-uniform in 1..100, Zipf(1.2), mean pooling, SGD lr 0.01
  5  1 fp16 table of 200M rows stored as 4 column slices of 32 (dim 128),
     batch 65536, hotness 20, Zipf(1.3), sum pooling, Adagrad

Keys are Zipf-distributed because categorical ids are frequency skewed; rank k
maps to row k-1, the order a frequency-sorted categorify step produces (NVIDIA
Merlin blog, NVTabular section: `Categorify(use_frequency=True)`). The 26-table
configurations echo the 26 categorical columns of the Criteo click logs named
on the same page; the dataset itself is not used, seeded synthetic keys stand
in for it.

Seeds: ``np.random.SeedSequence([cfg, stream, t, k])`` with stream 0 = sizes
and hotness, 1 = keys of table t, 2 = bag lengths of table t, 3 = upstream
gradient; k numbers the batch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

STREAM_SIZES = 0
STREAM_KEYS = 1
STREAM_LENGTHS = 2
STREAM_DY = 3

DTYPES = ("f32", "bf16", "f16")
DTYPE_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


def rng_for(cfg_id: int, stream: int, t: int = 0, k: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(stream), int(t), int(k)]))


# --------------------------------------------------------------------------
# Zipf sampler: rejection-inversion (Hoermann & Derflinger, 1996,
# "Rejection-inversion to generate variates from monotone discrete
# distributions"). Written from the method's description:
#   h(x) = x^-s is the (unnormalised) mass of rank x, H an antiderivative.
#   Draw V uniformly on [H(1.5) - h(1), H(n + 0.5)], X = H^-1(V), K = round(X).
#   The V-interval that rounds to K = k >= 2 is [H(k-.5), H(k+.5)), whose
#   length is >= h(k) because h is convex; accepting only the top h(k) of it
#   (V >= H(k+.5) - h(k)) makes P(K = k) proportional to h(k). For k = 1 the
#   interval has length exactly h(1), so it is always accepted.
# --------------------------------------------------------------------------

def _H(x: np.ndarray, s: float) -> np.ndarray:
    lx = np.log(x)
    if s == 1.0:
        return lx
    a = 1.0 - s
    return np.expm1(a * lx) / a


def _H_inv(y: np.ndarray, s: float) -> np.ndarray:
    if s == 1.0:
        return np.exp(y)
    a = 1.0 - s
    return np.exp(np.log1p(a * y) / a)


def zipf_ranks(rng: np.random.Generator, n: int, s: float, size: int) -> np.ndarray:
    """``size`` iid ranks in 1..n with P(k) proportional to k^-s (int64)."""
    if n < 1:
        raise ValueError("n must be >= 1")
    if n == 1:
        return np.ones(size, dtype=np.int64)
    lo = float(_H(np.array([1.5]), s)[0]) - 1.0
    hi = float(_H(np.array([n + 0.5]), s)[0])
    out = np.empty(size, dtype=np.int64)
    todo = np.arange(size)
    while todo.size:
        v = lo + rng.random(todo.size) * (hi - lo)
        x = _H_inv(v, s)
        k = np.clip(np.floor(x + 0.5), 1, n)
        ok = v >= _H(k + 0.5, s) - np.power(k, -s)
        ok |= k == 1
        out[todo[ok]] = k[ok].astype(np.int64)
        todo = todo[~ok]
    return out


# --------------------------------------------------------------------------
# Configurations
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class TableSpec:
    rows: int
    dim: int
    dtype: str = "f32"
    col_slices: int = 1


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    tables: tuple
    batch: int
    pool: str                  # "sum" | "mean"
    opt: str                   # "sgd" | "adagrad"
    lr: float
    eps: float
    hotness: tuple             # per table: int fixed length, or ("uniform", lo, hi)
    zipf_s: float | None       # None -> uniform keys
    init_seed: int = 0
    notes: str = ""

    @property
    def T(self) -> int:
        return len(self.tables)

    @property
    def dim(self) -> int:
        return self.tables[0].dim

    @property
    def dtype(self) -> str:
        return self.tables[0].dtype

    @property
    def total_rows(self) -> int:
        return int(sum(t.rows for t in self.tables))

    def row_offset(self) -> np.ndarray:
        ro = np.zeros(self.T + 1, dtype=np.int64)
        ro[1:] = np.cumsum([t.rows for t in self.tables])
        return ro


def _loguniform_int(rng, lo: float, hi: float, size: int) -> np.ndarray:
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size))).astype(np.int64)


def make_config(cfg_id: int, *, batch: int | None = None, num_tables: int | None = None,
                rows: int | None = None) -> Config:
    """Build configuration ``cfg_id`` (1..5). ``batch``/``num_tables``/``rows``
    shrink it for oracle-sized parity cases while keeping its structure."""
    if cfg_id == 1:
        rr = [1000, 5000, 10000, 50000]
        tabs = tuple(TableSpec(r, 16, "f32") for r in rr)
        cfg = Config(1, "tiny-4x16-f32-sgd", tabs, 128, "sum", "sgd", 0.01, 0.0,
                     tuple(("uniform", 1, 4) for _ in rr), None, init_seed=1)
    elif cfg_id == 2:
        rng = rng_for(2, STREAM_SIZES)
        rr = _loguniform_int(rng, 1e2, 1e6, 26)
        tabs = tuple(TableSpec(int(r), 64, "f32") for r in rr)
        cfg = Config(2, "26x-loguniform-x64-f32-adagrad", tabs, 16384, "sum", "adagrad", 0.01, 1e-8,
                     tuple(1 for _ in rr), 1.1, init_seed=2)
    elif cfg_id == 3:
        tabs = tuple(TableSpec(4_000_000, 128, "f32") for _ in range(26))
        cfg = Config(3, "26x4Mx128-f32-adagrad", tabs, 65536, "sum", "adagrad", 0.01, 1e-8,
                     tuple(1 for _ in range(26)), 1.05, init_seed=3)
    elif cfg_id == 4:
        rng = rng_for(4, STREAM_SIZES)
        hot = np.minimum(100, np.floor(np.exp(rng.uniform(0.0, math.log(101.0), 100)))).astype(np.int64)
        hot = np.maximum(hot, 1)
        tabs = tuple(TableSpec(1_000_000, 128, "bf16") for _ in range(100))
        cfg = Config(4, "100x1Mx128-bf16-sgd-mean", tabs, 32768, "mean", "sgd", 0.01, 0.0,
                     tuple(int(h) for h in hot), 1.2, init_seed=4)
    elif cfg_id == 5:
        tabs = (TableSpec(200_000_000, 128, "f16", 4),)
        cfg = Config(5, "1x200Mx(4x32)-f16-adagrad", tabs, 65536, "sum", "adagrad", 0.01, 1e-8,
                     (20,), 1.3, init_seed=5)
    else:
        raise ValueError(f"unknown config {cfg_id}")
    if num_tables is not None:
        cfg = replace(cfg, tables=cfg.tables[:num_tables], hotness=cfg.hotness[:num_tables])
    if rows is not None:
        cfg = replace(cfg, tables=tuple(replace(t, rows=min(t.rows, rows)) for t in cfg.tables))
    if batch is not None:
        cfg = replace(cfg, batch=int(batch))
    return cfg


# --------------------------------------------------------------------------
# Batches
# --------------------------------------------------------------------------

@dataclass
class Batch:
    indices: np.ndarray        # [N] int32 (or int64), row ids within each table
    offsets: np.ndarray        # [T*B + 1], table-major: bag (t, b) = offsets[t*B + b]
    lengths: np.ndarray        # [T*B] bag lengths
    T: int
    B: int

    @property
    def N(self) -> int:
        return int(self.indices.shape[0])


def bag_lengths(cfg: Config, t: int, k: int = 0) -> np.ndarray:
    h = cfg.hotness[t]
    if isinstance(h, tuple):
        _, lo, hi = h
        return rng_for(cfg.cfg_id, STREAM_LENGTHS, t, k).integers(lo, hi + 1, cfg.batch).astype(np.int64)
    return np.full(cfg.batch, int(h), dtype=np.int64)


def table_keys(cfg: Config, t: int, count: int, k: int = 0) -> np.ndarray:
    rng = rng_for(cfg.cfg_id, STREAM_KEYS, t, k)
    n = cfg.tables[t].rows
    if cfg.zipf_s is None:
        return rng.integers(0, n, count).astype(np.int64)
    return zipf_ranks(rng, n, cfg.zipf_s, count) - 1


def make_batch(cfg: Config, k: int = 0, index_dtype=np.int32) -> Batch:
    T, B = cfg.T, cfg.batch
    lengths = np.concatenate([bag_lengths(cfg, t, k) for t in range(T)]) if T else np.zeros(0, np.int64)
    idx = []
    for t in range(T):
        cnt = int(lengths[t * B:(t + 1) * B].sum())
        idx.append(table_keys(cfg, t, cnt, k))
    indices = np.concatenate(idx) if idx else np.zeros(0, np.int64)
    offsets = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    return Batch(indices.astype(index_dtype), offsets.astype(index_dtype), lengths, T, B)


def make_batch_from_lengths(lengths_per_table, keys_per_table, B: int, index_dtype=np.int32) -> Batch:
    """Assemble an explicit CSR batch (edge-case tests): ``lengths_per_table[t]``
    has B bag lengths, ``keys_per_table[t]`` their concatenated row ids."""
    T = len(lengths_per_table)
    lengths = np.concatenate([np.asarray(l, np.int64) for l in lengths_per_table]) if T else np.zeros(0, np.int64)
    keys = [np.asarray(k, np.int64) for k in keys_per_table]
    for t in range(T):
        assert keys[t].shape[0] == int(np.asarray(lengths_per_table[t]).sum())
    indices = np.concatenate(keys) if keys else np.zeros(0, np.int64)
    offsets = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    return Batch(indices.astype(index_dtype), offsets.astype(index_dtype), lengths, T, B)


def make_dy(cfg: Config, k: int = 0) -> np.ndarray:
    """Upstream gradient dL/dY, N(0, 1) fp32, shape [B, T*D]."""
    rng = rng_for(cfg.cfg_id, STREAM_DY, 0, k)
    return rng.standard_normal((cfg.batch, cfg.T * cfg.dim), dtype=np.float32)


def make_int_dy(cfg: Config, k: int = 0, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integer-valued upstream gradient in [lo, hi] (fp32). With sum pooling
    every fp32 partial sum of such values is exact, whatever the order."""
    rng = rng_for(cfg.cfg_id, STREAM_DY, 1, k)
    return rng.integers(lo, hi + 1, (cfg.batch, cfg.T * cfg.dim)).astype(np.float32)
