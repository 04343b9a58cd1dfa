"""GPU parity of the unique-first forward (emb_forward_pooled_unique): every
unique row gathered once, bags pooled from the compact rows through the
inverse. The output must equal emb_forward_pooled's bit for bit (same rows,
same order of additions) and so the oracle's within the forward tolerance."""
import gc

import numpy as np
import pytest
import torch

from dlrm_sparse_embedding_amd import workloads as W

from tests import parity as P

pytestmark = pytest.mark.gpu

REDUCED = {1: dict(), 2: dict(batch=2048), 3: dict(batch=1024), 4: dict(batch=48), 5: dict(batch=1024, rows=2_000_000)}


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _same(Y0, Y1):
    bad = Y0.view(np.uint32) != Y1.view(np.uint32)
    if bad.any():
        r, c = np.nonzero(bad)
        raise AssertionError(f"{int(bad.sum())} of {bad.size} differ; first (sample, col, direct, unique): "
                             f"{[(int(a), int(b), float(Y0[a, b]), float(Y1[a, b])) for a, b in zip(r[:8], c[:8])]}")


def _both(cfg, batch, dY, pool=None):
    pool = pool or cfg.pool
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, dY)
    B, N = cfg.batch, batch.N
    Y0 = tabs.forward(idx, off, B, pool)
    bufs = tabs.backward_buffers(N, B, with_grad=False)
    tabs.dedup(idx, off, B, pool, bufs)
    rows = tabs.unique_rows_buffer(N)
    Y1 = tabs.forward_unique(idx, off, B, pool, bufs, rows)
    torch.cuda.synchronize()
    return tabs, (idx, off, dy), bufs, Y0.cpu().numpy(), Y1.cpu().numpy()


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_unique_forward_equals_direct_and_oracle(cfg_id):
    cfg = W.make_config(cfg_id, **REDUCED[cfg_id])
    batch = W.make_batch(cfg, k=1)
    dY = W.make_dy(cfg, k=1)
    P.say("unique forward", cfg_id, "N", batch.N)
    tabs, _, _, Y0, Y1 = _both(cfg, batch, dY)
    _same(Y0, Y1)
    P.check_forward(Y1, cfg, batch, P.oracle_tables(cfg, batch))
    tabs.close()


@pytest.mark.parametrize("pool", ["sum", "mean"])
def test_unique_forward_ragged_and_bad_indices(pool):
    rng = np.random.default_rng(4)
    cfg = P.custom_cfg([1, 7, 300, 5000], dim=32, B=333, pool=pool)
    lens = [rng.integers(0, 6, cfg.batch) * (rng.random(cfg.batch) < 0.7) for _ in range(cfg.T)]
    lens[1][:] = 0
    keys = [rng.integers(0, cfg.tables[t].rows, int(lens[t].sum())) for t in range(cfg.T)]
    keys[2][:5] = 300                                        # out of range for table 2
    batch = W.make_batch_from_lengths(lens, keys, cfg.batch, index_dtype=np.int64)
    dY = rng.standard_normal((cfg.batch, cfg.T * cfg.dim)).astype(np.float32)
    P.say("unique forward ragged", pool)
    tabs, _, _, Y0, Y1 = _both(cfg, batch, dY)
    _same(Y0, Y1)
    with pytest.raises(Exception):
        tabs.check_device_error()
    tabs.close()


def test_backward_after_unique_forward():
    # the dedup done ahead serves both the unique-first forward and the
    # backward + fused update, which then match the plain path bit for bit
    cfg = W.make_config(2, batch=2048)
    batch = W.make_batch(cfg, k=4)
    dY = W.make_dy(cfg, k=4)
    u, _, _ = P.oracle_dedup(cfg, batch)
    P.say("backward after unique forward cfg2")
    tabs, (idx, off, dy), bufs, Y0, Y1 = _both(cfg, batch, dY)
    tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs)
    tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs, dY=dy)
    torch.cuda.synchronize()
    w1, G1 = P.read_rows(tabs, cfg, u)
    tabs.close()
    ref = P.run_step(cfg, batch, dY, sample_untouched=0)
    assert np.array_equal(w1.view(np.uint32), ref["w_new"].view(np.uint32))
    assert np.array_equal(G1.view(np.uint32), ref["G_new"].view(np.uint32))


@pytest.mark.slow
@pytest.mark.parametrize("cfg_id", [3, 5])
def test_unique_forward_full_size(cfg_id):
    cfg = W.make_config(cfg_id)
    batch = W.make_batch(cfg, k=2)
    P.say("unique forward full", cfg_id, "N", batch.N)
    tabs, _, _, Y0, Y1 = _both(cfg, batch, None)
    _same(Y0, Y1)
    tabs.close()
