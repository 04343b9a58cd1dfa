"""Multi-hot batches (more lookups than bags): segment lengths around the
chunk (128), level-1 tile (4096) and 256-position marks, a key repeated inside
one bag, batches of fewer bags than the reduce has XCDs, integer gradients
(exact sums, bit-exact rows), fused == materialised bit for bit, and chunk
lists of one to a few chunks. Every element is checked against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
from tests import parity as P
from dlrm_sparse_embedding_amd import workloads as W

pytestmark = pytest.mark.gpu

TILE = 4096      # level-1 tile of the sorted positions
LONG = 256


def _say(*a):
    print("[case]", *a, flush=True)


def _fill(counts, upto, rng):
    """Append keys of 1 or 2 lookups until the sorted position reaches `upto`."""
    pos = int(sum(counts))
    assert pos <= upto
    while pos < upto:
        c = 1 if upto - pos == 1 else int(rng.integers(1, 3))
        counts.append(c)
        pos += c


def _boundary_counts(rng):
    """Lookup counts per key (key k = k-th entry), in key order, so that
    segment k starts at the sum of the counts before it."""
    c = [255, 256, 257, 1, 2, 3]          # around two chunks
    _fill(c, TILE, rng)
    c.append(5000)                        # starts exactly at tile 1, ends in tile 2
    c += [300, 300, 300]                  # three long segments starting in one tile
    _fill(c, 4 * TILE - 700, rng)
    c.append(700)                         # ends exactly at the start of tile 4
    _fill(c, 5 * TILE - 100, rng)
    c.append(200)                         # short, crosses into tile 5
    c.append(2 * TILE + 1)                # spans three tiles
    c += [LONG - 1] * 3
    _fill(c, 8 * TILE + 37, rng)          # a ragged last tile
    return np.asarray(c, np.int64)


def _batch_from_counts(counts, L, rng):
    keys = np.repeat(np.arange(len(counts)), counts)
    rng.shuffle(keys)
    n = len(keys)
    B = n // L
    keys = keys[: B * L]
    lens = np.full(B, L)
    return W.make_batch_from_lengths([lens], [keys], B), B


def _cfg(rows, dim, dtype, B, pool, opt, slices=1):
    tabs = (W.TableSpec(rows, dim, dtype, slices),)
    return W.Config(98, "multi-hot-edges", tabs, B, pool, opt, 0.05, 1e-8, (1,), None, init_seed=98)


@pytest.mark.parametrize("dim,dtype,pool,opt,L", [(128, "f32", "sum", "adagrad", 8),
                                                  (64, "bf16", "mean", "sgd", 5),
                                                  (128, "f16", "sum", "adagrad", 3)])
def test_segment_lengths_and_tile_edges(dim, dtype, pool, opt, L):
    rng = np.random.default_rng(17)
    counts = _boundary_counts(rng)
    batch, B = _batch_from_counts(counts, L, rng)
    cfg = _cfg(len(counts) + 10, dim, dtype, B, pool, opt, slices=2 if dtype == "f16" else 1)
    assert batch.N > cfg.T * B
    dY = rng.standard_normal((B, dim)).astype(np.float32)
    _say("tile edges", dim, dtype, pool, opt, L, "N", batch.N, "B", B)
    for path in ("materialized", "fused"):
        P.run_step(cfg, batch, dY, path=path)


@pytest.mark.parametrize("B", [1, 3, 7])
def test_few_long_bags(B):
    # a few long bags: every segment repeats bags, chunks run to 128 positions
    rng = np.random.default_rng(23 + B)
    L = 1500
    keys = []
    for b in range(B):
        k = rng.integers(0, 40, L)
        k[: L // 3] = 5                      # one hot key in every bag
        keys.append(k)
    batch = W.make_batch_from_lengths([np.full(B, L)], [np.concatenate(keys)], B)
    cfg = _cfg(64, 32, "f32", B, "mean", "adagrad")
    dY = rng.standard_normal((B, 32)).astype(np.float32)
    _say("few bags", B)
    for path in ("materialized", "fused"):
        P.run_step(cfg, batch, dY, path=path)


def test_integer_grad_bit_exact_over_tile_edges():
    # exact sums: the stored rows must equal the oracle's bit for bit, long
    # segments (chunk partials + combine) and short ones alike
    rng = np.random.default_rng(29)
    counts = _boundary_counts(rng)
    batch, B = _batch_from_counts(counts, 6, rng)
    cfg = _cfg(len(counts) + 4, 64, "bf16", B, "sum", "sgd")
    from dataclasses import replace
    cfg = replace(cfg, lr=2.0 ** -7)
    dY = rng.integers(-8, 9, (B, 64)).astype(np.float32)
    _say("int-grad tile edges N", batch.N)
    tabs = P.make_tables(cfg, master=True)
    r = P.run_step(cfg, batch, dY, path="fused", tabs=tabs, master=True)
    u, c, inv = P.oracle_dedup(cfg, batch)
    g = O.reduced_grad(dY, batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool, inv, len(u))
    assert np.all(np.abs(g) < 2 ** 24)
    m_ref, w_ref, _ = O.update_rows_master(P.stored_init(cfg, u, rounded=False), None, g, "sgd", cfg.lr,
                                           cfg.eps, cfg.dtype)
    assert np.array_equal(P.read_master(tabs, cfg, u).view(np.uint32), m_ref.view(np.uint32))
    assert np.array_equal(r["w_new"].view(np.uint32), w_ref.view(np.uint32))
    tabs.close()


def test_fused_equals_materialized_and_reruns_bit_identical():
    # the workload of 1 fp16 table x (4 x 32) columns, 20 lookups per bag,
    # Zipf 1.3, at a reduced batch: same bits from both paths and on a rerun
    cfg = W.make_config(5, rows=2_000_000, batch=4096)
    batch = W.make_batch(cfg, k=2)
    dY = W.make_dy(cfg, k=2)
    _say("multi-hot determinism N", batch.N)
    res = [P.run_step(cfg, batch, dY, path=p, sample_untouched=0) for p in ("fused", "materialized", "fused")]
    for r in res[1:]:
        assert np.array_equal(r["w_new"].view(np.uint32), res[0]["w_new"].view(np.uint32))
        assert np.array_equal(r["G_new"].view(np.uint32), res[0]["G_new"].view(np.uint32))



@pytest.mark.parametrize("pool,itype", [("sum", np.int32), ("mean", np.int64)])
def test_long_bags_out_of_range_in_later_index_blocks(pool, itype):
    # bags of up to 150 lookups: the forward reads their row indices 16 (or
    # 32) at a time, one block ahead; out-of-range indices sit in later
    # blocks too. They add nothing, count in a mean's length, set the bounds
    # flag, and every other element still matches the oracle.
    import torch
    from dlrm_sparse_embedding_amd import emb as E
    rng = np.random.default_rng(31)
    rows = [5000, 300]
    tabs_spec = tuple(W.TableSpec(r, 64, "bf16") for r in rows)
    B = 96
    cfg = W.Config(97, "long-bags", tabs_spec, B, pool, "sgd", 0.05, 0.0, (1, 1), None, init_seed=97)
    lens = [rng.integers(0, 151, B), rng.integers(15, 40, B)]
    keys = []
    for t, r in enumerate(rows):
        k = rng.integers(0, r, int(lens[t].sum()))
        bad = rng.random(len(k)) < 0.02
        k[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, r + 3)
        keys.append(k)
    batch = W.make_batch_from_lengths(lens, keys, B, index_dtype=itype)
    _say("long bags out of range", pool, itype.__name__, "N", batch.N)
    tabs = P.make_tables(cfg)
    idx, off, _ = P.to_dev(batch, None)
    Y = tabs.forward(idx, off, B, pool)
    torch.cuda.synchronize()
    with pytest.raises(E.EmbError) as ei:
        tabs.check_device_error()
    assert ei.value.code == E.EMB_E_BOUNDS
    P.check_forward(Y.cpu().numpy(), cfg, batch, P.oracle_tables(cfg, batch), num_rows=rows)
    tabs.close()


def test_fused_equals_materialized_bf16_mean_sgd():
    # the 100-table bf16 workload's arithmetic (mean pooling, SGD, 1..93
    # lookups per bag by table) on 12 tables at a reduced batch
    cfg = W.make_config(4, num_tables=12, batch=512)
    batch = W.make_batch(cfg, k=1)
    dY = W.make_dy(cfg, k=1)
    _say("multi-hot determinism bf16 N", batch.N)
    res = [P.run_step(cfg, batch, dY, path=p, sample_untouched=0) for p in ("fused", "materialized", "fused")]
    for r in res[1:]:
        assert np.array_equal(r["w_new"].view(np.uint32), res[0]["w_new"].view(np.uint32))


@pytest.mark.parametrize("dim,dtype,opt,case", [(128, "f32", "adagrad", "one"), (128, "f32", "adagrad", "two"),
                                                (128, "f32", "sgd", "three"), (256, "bf16", "sgd", "odd"),
                                                (128, "f32", "adagrad", "repeat")])
def test_short_chunk_lists(dim, dtype, opt, case):
    # a handful of chunks: the reduce's waves read their next descriptors in
    # pairs from a clamped base, so lists of 1, 2, 3 and an odd number of
    # chunks (and a wave whose second chunk lies past the end) must still
    # give every key its own sum
    rng = np.random.default_rng(41)
    rows = 50
    if case == "one":
        lens, keys = [np.array([1])], [np.array([7])]
    elif case == "two":
        lens, keys = [np.array([1, 1])], [np.array([7, 9])]
    elif case == "three":
        lens, keys = [np.array([2, 1, 0])], [np.array([3, 7, 7])]
    elif case == "odd":
        lens = [rng.integers(0, 4, 9)]
        keys = [rng.integers(0, rows, int(lens[0].sum()))]
    else:  # one key in every bag, several times: one segment split into chunks only at tile edges
        lens = [np.full(5, 3)]
        keys = [np.full(15, 11)]
    B = len(lens[0])
    batch = W.make_batch_from_lengths(lens, keys, B)
    cfg = _cfg(rows, dim, dtype, B, "sum", opt)
    dY = rng.standard_normal((B, dim)).astype(np.float32)
    _say("short chunk list", case, dim, dtype, opt, "N", batch.N)
    for path in ("materialized", "fused"):
        P.run_step(cfg, batch, dY, path=path)
