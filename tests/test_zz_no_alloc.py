"""GPU test of emb_hash_translate_noalloc, the id -> row translation that
allocates nothing (its scratch is the library's fixed per-GPU array): two
contexts with identical maps translate the same batches, one through
emb_hash_translate with a caller workspace and one through the no-allocation
entry point, and every row handed out, and every table's count of rows used,
must agree bit for bit -- on consecutive calls, the later ones smaller than
the first (the fixed array keeps the earlier call's contents), with insertion
and lookup-only. Both are also checked against the oracle's HashTables."""
import gc

import numpy as np
import pytest
import torch

import oracle as O
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


def _ids(rng, rows, B, hot, universe, index_dtype):
    T = len(rows)
    lens = [rng.integers(0, 2 * hot + 1, B) for _ in range(T)]
    ids = []
    for t in range(T):
        ranks = np.minimum(rng.zipf(1.2, int(lens[t].sum())), universe) - 1
        x = (ranks.astype(np.uint64) * np.uint64(0x9E3779B97F4A7C15)) ^ np.uint64(t * 0x2545F4914F6CDD1D + 3)
        ids.append(x.view(np.int64))
    batch = W.make_batch_from_lengths(lens, [np.zeros(int(l.sum()), np.int64) for l in lens], B,
                                      index_dtype=index_dtype)
    return batch, np.concatenate(ids)


@pytest.mark.parametrize("index_dtype", [np.int32, np.int64])
def test_noalloc_translate_matches_workspace_translate(index_dtype):
    rng = np.random.default_rng(21)
    rows = [3000, 50_000, 40, 200_000]             # table 2 fills up
    cfg = P.custom_cfg(rows, dim=16, B=40_000)
    P.say("no-alloc translate", index_dtype.__name__)
    ta, tb = P.make_tables(cfg), P.make_tables(cfg)
    ta.hash_attach()
    tb.hash_attach()
    ht = O.HashTables(rows)
    # consecutive calls: a large one (about 1.2 M lookups), then smaller ones
    plan = [(40_000, 8, True), (700, 3, True), (5_000, 2, False), (64, 1, True)]
    for step, (B, hot, insert) in enumerate(plan):
        batch, ids = _ids(rng, rows, B, hot, 400_000, index_dtype)
        d_ids = torch.from_numpy(ids).cuda()
        d_off = torch.from_numpy(batch.offsets).cuda()
        ra = ta.hash_translate(d_ids, d_off, B, insert)
        rb = torch.full_like(ra, -7)
        E.emb_hash_translate_noalloc(tb.ctx, d_ids, d_off, B, insert, rb)
        torch.cuda.synchronize()
        got_a = ra.cpu().numpy().astype(np.int64)
        got_b = rb.cpu().numpy().astype(np.int64)
        ref = ht.translate(ids, batch.offsets, cfg.T, B, insert)
        assert np.array_equal(got_b, got_a), (step, int((got_a != got_b).sum()))
        assert np.array_equal(got_b, ref), (step, int((got_b != ref).sum()))
        assert ta.hash_rows_used().cpu().tolist() == tb.hash_rows_used().cpu().tolist() == ht.next_free
    ta.check_device_error()
    tb.check_device_error()
    ta.close()
    tb.close()


def test_noalloc_translate_rejects_oversize_and_empty():
    cfg = P.custom_cfg([100], dim=16, B=4)
    P.say("no-alloc translate limits")
    tabs = P.make_tables(cfg)
    with pytest.raises(E.EmbError) as ei:              # no map memory attached yet
        E.emb_hash_translate_noalloc(tabs.ctx, torch.zeros(4, dtype=torch.int64, device="cuda"),
                                     torch.arange(5, dtype=torch.int32, device="cuda"), 4, True,
                                     torch.empty(4, dtype=torch.int32, device="cuda"))
    assert ei.value.code == E.EMB_E_STATE
    tabs.hash_attach()
    # more lookups than the fixed scratch holds: rejected before any launch
    N = 2_000_000
    assert E.emb_hash_workspace_bytes(tabs.ctx, N) > 64 << 20
    ids = torch.zeros(N, dtype=torch.int64, device="cuda")
    off = torch.tensor([0, N // 2, N // 2, N, N], dtype=torch.int32, device="cuda")
    rows = torch.empty(N, dtype=torch.int32, device="cuda")
    with pytest.raises(E.EmbError) as ei:
        E.emb_hash_translate_noalloc(tabs.ctx, ids, off, 4, True, rows)
    assert ei.value.code == E.EMB_E_WORKSPACE
    # no lookups: nothing to do
    E.emb_hash_translate_noalloc(tabs.ctx, ids[:0], torch.zeros(5, dtype=torch.int32, device="cuda"), 4, True,
                                 rows[:0])
    torch.cuda.synchronize()
    tabs.check_device_error()
    tabs.close()
