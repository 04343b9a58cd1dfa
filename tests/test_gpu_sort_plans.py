"""The dedup's radix sort under each of its plans, through the whole step
(forward, dedup, reduce, fused or materialised update) against the oracle.

The library sorts either globally (one segment, the key's own bits) or per
table (each table's contiguous positions on its row bits), with digits of 8
to 10 bits: per table when that needs fewer passes, or as many passes with
narrower digits. The cases below pin each plan and
digit width, ragged and empty bags, a table without lookups (an empty
segment), and out-of-range indices under the per-table plan.
"""
import gc
import zlib

import numpy as np
import pytest
import torch

from dlrm_sparse_embedding_amd import emb as E
from dlrm_sparse_embedding_amd import workloads as W

from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bits(x):
    b = 1
    while (1 << b) <= x:
        b += 1
    return b


def _plan(rows):
    """(per-table?, passes, digit bits) the library picks for these tables."""
    def one(bits):
        p = 1 if bits <= 10 else -(-bits // 10)
        return p, min(10, max(8, -(-bits // p)))
    glob, seg = one(_bits(sum(rows))), one(_bits(max(rows)))
    if len(rows) <= 256 and seg < glob:      # fewer passes, or as many with narrower digits
        return (True,) + seg
    return (False,) + glob


def _batch(rng, rows, B, maxlen, s=1.2, empty_table=None, itype=np.int32):
    lens = [rng.integers(0, maxlen + 1, B) * (rng.random(B) < 0.9) if maxlen > 1 else np.ones(B, int)
            for _ in rows]
    if empty_table is not None:
        lens[empty_table][:] = 0
    keys = [np.minimum(W.zipf_ranks(rng, r, s, int(l.sum())), r) - 1 for l, r in zip(lens, rows)]
    return W.make_batch_from_lengths(lens, keys, B, index_dtype=itype)


CASES = {
    # name: rows, B, max bag length, dim, expected plan
    "table_1pass_10bit": ([1000, 700, 1023, 10, 500, 999], 700, 4, 16, (True, 1, 10)),
    "table_2pass_10bit": ([1_000_000, 900_000, 1000, 1_000_000, 1_000_000, 600_000, 20], 3000, 5, 16, (True, 2, 10)),
    "table_3pass_8bit": ([4_000_000, 5000, 4_000_000, 4_000_000, 4_000_000, 4_000_000], 4096, 3, 16, (True, 3, 8)),
    "global_2pass_8bit": ([5000], 2000, 6, 32, (False, 2, 8)),
    "global_2pass_10bit": ([600_000], 3000, 4, 16, (False, 2, 10)),
    "global_3pass_8bit": ([3_000_000], 3000, 4, 16, (False, 3, 8)),
    "global_3pass_10bit": ([200_000_000], 2048, 3, 16, (False, 3, 10)),
}


def test_sort_plan_large_tiles():
    # sorts of >= 16 Mi items use 4096-item tiles: 8 tables x 1M rows (per
    # table, 2 passes of 10 bits), 65536 samples x 32 lookups = 16 Mi lookups
    rows = [1_000_000] * 8
    assert _plan(rows) == (True, 2, 10)
    B, h = 65536, 32
    rng = np.random.default_rng(5)
    lens = [np.full(B, h, int) for _ in rows]
    keys = [np.minimum(W.zipf_ranks(rng, r, 1.2, B * h), r) - 1 for r in rows]
    batch = W.make_batch_from_lengths(lens, keys, B)
    assert batch.N >= 16 << 20
    cfg = P.custom_cfg(rows, dim=16, B=B, pool="mean", opt="sgd")
    dY = rng.standard_normal((B, len(rows) * 16)).astype(np.float32)
    P.say("sort plan, large tiles", "N", batch.N)
    P.run_step(cfg, batch, dY, path="fused", sample_bags=256, sample_keys=2000, sample_untouched=500)


@pytest.mark.parametrize("name", sorted(CASES))
def test_sort_plan_step(name):
    rows, B, maxlen, dim, want = CASES[name]
    assert _plan(rows) == want, (name, _plan(rows))
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    cfg = P.custom_cfg(rows, dim=dim, B=B, pool="sum", opt="adagrad")
    batch = _batch(rng, rows, B, maxlen, empty_table=len(rows) - 1 if len(rows) > 2 else None,
                   itype=np.int64 if "10bit" in name else np.int32)
    dY = rng.standard_normal((B, len(rows) * dim)).astype(np.float32)
    path = "materialized" if "1pass" in name else "fused"
    P.say("sort plan", name, "rows", rows, "B", B, "N", batch.N, path)
    P.run_step(cfg, batch, dY, path=path, sample_keys=4000, sample_untouched=500)


def test_table_plan_out_of_range_indices():
    # per-table plan: a lookup whose index is out of range gets the sentinel
    # key sum(rows), which sorts after its own table's keys and is never
    # applied; every in-range lookup is reduced and applied as without it
    rows = [1000, 700, 1023, 10, 500, 999]
    assert _plan(rows)[0]
    rng = np.random.default_rng(7)
    B = 256
    cfg = P.custom_cfg(rows, dim=16, B=B, pool="sum", opt="sgd")
    keys = [rng.integers(0, r, B) for r in rows]
    keys[1][[3, 50, 200]] = [700, -1, 99999]
    keys[3][7] = 10
    batch = W.make_batch_from_lengths([np.ones(B, int)] * len(rows), keys, B, index_dtype=np.int64)
    P.say("table plan, out-of-range indices")
    tabs = P.make_tables(cfg)
    dY = np.ones((B, len(rows) * 16), np.float32)
    idx, off, dy = P.to_dev(batch, dY)
    bufs = tabs.backward_buffers(batch.N, B, with_grad=False)
    tabs.backward(idx, off, B, "sum", dy, bufs)
    tabs.update("sgd", 0.5, 0.0, bufs, dY=dy)
    with pytest.raises(E.EmbError) as ei:
        tabs.check_device_error()
    assert ei.value.code == E.EMB_E_BOUNDS
    U = int(bufs["num_unique"].item())
    uk = bufs["unique_keys"][:U].cpu().numpy().view(np.uint32).astype(np.int64)
    cnt = bufs["counts"][:U].cpu().numpy().astype(np.int64)
    inv = bufs["inverse"][:batch.N].cpu().numpy().astype(np.int64)
    ro = cfg.row_offset()
    g = np.concatenate([np.where((k >= 0) & (k < r), ro[t] + k, cfg.total_rows)
                        for t, (k, r) in enumerate(zip(keys, rows))])
    assert np.array_equal(uk[inv], g)                         # every lookup's key
    assert np.array_equal(np.bincount(inv, minlength=U), cnt)  # counts
    valid = uk[uk != cfg.total_rows]
    assert np.all(np.diff(valid) > 0)                         # in-range keys: ascending, unique
    assert np.array_equal(valid, np.unique(g[g != cfg.total_rows]))
    assert 1 <= (uk == cfg.total_rows).sum() <= 2               # one sentinel run per table holding one
    # in-range rows moved by -0.5 * (their lookup count) per column; the rest are untouched
    w, _ = P.read_rows(tabs, cfg, np.arange(cfg.total_rows))
    init = P.stored_init(cfg, np.arange(cfg.total_rows))
    mult = np.bincount(g[g != cfg.total_rows], minlength=cfg.total_rows).astype(np.float32)
    ref = (init - np.float32(0.5) * mult[:, None]).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))
    tabs.close()


LENGTH_CASES = {
    # name: rows, B, bag lengths per table (an int: every bag; a list: a pattern repeated)
    "one_hot": ([3000, 700, 1999], 1000, [1, 1, 1]),
    "fixed_hotness": ([3000, 700, 1999, 50], 1000, [3, 1, 7, 2]),
    "pairs_and_empties": ([3000, 700, 1999], 1000, [1, [0, 2], 1]),   # N == T*B, not one lookup per bag
    "one_odd_bag_last": ([3000, 700, 1999], 1000, [1, 1, "last2"]),   # N == T*B + 1
    "empty_table": ([3000, 700, 1999], 1000, [2, 0, 2]),
    "straddling_groups": ([3000, 700, 1999, 800], 1000 - 37, [1, 1, 1, 1]),   # B % 64 != 0
    "many_tables_per_group": ([300, 70, 199, 80, 90], 13, [1, 1, 1, 1, 1]),  # B < 32
}


@pytest.mark.parametrize("rows", [[1000, 700, 1023, 10, 500, 999], [50, 60, 40]], ids=["table_plan", "global_plan"])
def test_multi_hot_out_of_range_inverse(rows):
    # ragged multi-hot bags (not one lookup per bag, so the inverse goes
    # through the key -> segment map) with out-of-range indices in several
    # tables: every lookup's inverse names a segment holding its own key, the
    # sentinel sum(rows) for the bad ones (one run per table under the
    # per-table plan, one run for all tables under the global plan), and the
    # counts add up
    want_table = rows[0] == 1000
    assert _plan(rows)[0] == want_table
    rng = np.random.default_rng(11)
    B = 300
    lens = [rng.integers(0, 6, B) for _ in rows]
    keys = [rng.integers(0, r, int(l.sum())) for l, r in zip(lens, rows)]
    for t in (0, 1, len(rows) - 1):          # bad indices in three tables
        k = keys[t]
        k[rng.choice(len(k), 3, replace=False)] = [rows[t], -1, 10 * rows[t] + 7]
    batch = W.make_batch_from_lengths(lens, keys, B, index_dtype=np.int64)
    assert batch.N > len(rows) * B // 2
    cfg = P.custom_cfg(rows, dim=16, B=B, pool="mean", opt="sgd")
    P.say("multi-hot out-of-range inverse", "table plan" if want_table else "global plan", "N", batch.N)
    tabs = P.make_tables(cfg)
    dY = np.ones((B, len(rows) * 16), np.float32)
    idx, off, dy = P.to_dev(batch, dY)
    bufs = tabs.backward_buffers(batch.N, B, with_grad=False)
    tabs.backward(idx, off, B, "mean", dy, bufs)
    tabs.update("sgd", 0.5, 0.0, bufs, dY=dy)
    with pytest.raises(E.EmbError) as ei:
        tabs.check_device_error()
    assert ei.value.code == E.EMB_E_BOUNDS
    U = int(bufs["num_unique"].item())
    uk = bufs["unique_keys"][:U].cpu().numpy().view(np.uint32).astype(np.int64)
    cnt = bufs["counts"][:U].cpu().numpy().astype(np.int64)
    inv = bufs["inverse"][:batch.N].cpu().numpy().astype(np.int64)
    ro = cfg.row_offset()
    g = np.concatenate([np.where((k >= 0) & (k < r), ro[t] + k, cfg.total_rows)
                        for t, (k, r) in enumerate(zip(keys, rows))])
    assert inv.min() >= 0 and inv.max() < U
    assert np.array_equal(uk[inv], g)                          # every lookup's key
    assert np.array_equal(np.bincount(inv, minlength=U), cnt)  # counts
    in_range = uk[uk < cfg.total_rows]
    assert np.array_equal(in_range, np.unique(g[g < cfg.total_rows]))  # distinct, ascending
    n_sent = int((uk == cfg.total_rows).sum())
    assert n_sent == (3 if want_table else 1)
    tabs.close()


@pytest.mark.parametrize("name", sorted(LENGTH_CASES))
def test_bag_of_position(name):
    # the sort word carries each lookup's bag; the encoder stores the inverse
    # at the bag only when every bag holds exactly one lookup at its own index,
    # and goes through the key -> segment map otherwise (N == T*B alone must not
    # take the direct store); mean pooling weights each lookup by 1/L, so a
    # wrong bag shows up in the reduced gradient, and a wrong inverse in the
    # dedup check
    rows, B, spec = LENGTH_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lens = []
    for r in spec:
        if isinstance(r, int):
            lens.append(np.full(B, r, int))
        elif r == "last2":
            l = np.ones(B, int)
            l[-1] = 2
            lens.append(l)
        else:
            lens.append(np.resize(np.array(r, int), B))
    keys = [np.minimum(W.zipf_ranks(rng, r, 1.1, int(l.sum())), r) - 1 for l, r in zip(lens, rows)]
    batch = W.make_batch_from_lengths(lens, keys, B)
    cfg = P.custom_cfg(rows, dim=16, B=B, pool="mean", opt="adagrad")
    dY = rng.standard_normal((B, len(rows) * 16)).astype(np.float32)
    P.say("bag of position", name, "B", B, "N", batch.N)
    P.run_step(cfg, batch, dY, path="materialized", sample_untouched=500)
