"""GPU parity of the shard routing (emb_set_shard_map / emb_pack_by_shard)
against the oracle's pack_by_shard: keys, offsets and slots bit-exact; the
reduced gradients written into their send slots equal, bit for bit, the ones
emb_backward_unique_reduce writes in unique-key order, and the oracle's within
the fp32 tolerance."""
import gc

import numpy as np
import pytest
import torch

import oracle as O
from dlrm_sparse_embedding_amd import workloads as W

from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rules(kind_of, T, S):
    out = []
    for t in range(T):
        k = kind_of(t)
        out.append((k, 0 if k == O.SHARD_ROW_BLOCK else (7 * t + 1) % S))
    return out


def _run_pack(cfg, batch, dY, rules, S, unique_ref=None, grad=True):
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, dY)
    N, B = batch.N, cfg.batch
    bufs = tabs.backward_buffers(N, B, with_grad=True)
    tabs.backward(idx, off, B, cfg.pool, dy, bufs)            # reduced gradient in unique-key order
    tabs.set_shard_map(rules, S)
    pb = tabs.pack_buffers(N, S, with_grad=grad)
    tabs.pack(bufs, pb, dY=dy if grad else None)
    torch.cuda.synchronize()
    U = int(bufs["num_unique"].item())
    uk = bufs["unique_keys"][:U].cpu().numpy().view(np.uint32).astype(np.int64)
    if unique_ref is None:
        u, c, inv = P.oracle_dedup(cfg, batch)
        assert np.array_equal(uk, u)
    else:
        u, inv = unique_ref, None
        assert np.array_equal(uk, u)
    ok, ooff, oslot, _ = O.pack_by_shard(u, cfg.row_offset(), rules, S)
    nsend = int(ooff[-1])
    got_off = pb["send_offsets"].cpu().numpy().astype(np.int64)
    assert np.array_equal(got_off, ooff), "send offsets differ"
    got_keys = pb["send_keys"][:nsend].cpu().numpy().view(np.uint32).astype(np.int64)
    assert np.array_equal(got_keys, ok), "send keys differ"
    got_slot = pb["slot_of_unique"][:U].cpu().numpy().astype(np.int64)
    assert np.array_equal(got_slot, oslot), "slots differ"
    if grad and nsend:
        valid = np.nonzero(oslot >= 0)[0]
        sg = pb["send_grad"][:nsend].cpu().numpy()
        rg = bufs["reduced_grad"][:U].cpu().numpy()
        # the same reduction order: bit-identical to the unique-order output
        assert np.array_equal(sg[oslot[valid]].view(np.uint32), rg[valid].view(np.uint32))
        if inv is not None:
            g_ref, m_ref = P.grad_bounds(cfg, batch, dY, inv, U)
            P.check_grad(sg[oslot[valid]], g_ref[valid], m_ref[valid])
    return tabs, bufs, pb, dy


@pytest.mark.parametrize("cfg_id,S,kinds", [
    (2, 8, "mixed"), (2, 1, "cyclic"), (3, 4096, "cyclic"), (3, 512, "mixed"), (3, 511, "table"),
    (4, 64, "block"), (5, 3, "block"), (5, 37, "cyclic")])
def test_pack_matches_oracle(cfg_id, S, kinds):
    kw = dict(P_REDUCED[cfg_id])
    cfg = W.make_config(cfg_id, **kw)
    kind_of = {"mixed": lambda t: t % 3, "cyclic": lambda t: O.SHARD_ROW_CYCLIC,
               "table": lambda t: O.SHARD_TABLE, "block": lambda t: O.SHARD_ROW_BLOCK}[kinds]
    rules = _rules(kind_of, cfg.T, S)
    batch = W.make_batch(cfg, k=2)
    dY = W.make_dy(cfg, k=2)
    P.say("pack", cfg_id, S, kinds, "N", batch.N)
    tabs, *_ = _run_pack(cfg, batch, dY, rules, S)
    tabs.close()


P_REDUCED = {2: dict(batch=2048), 3: dict(batch=1024), 4: dict(batch=48), 5: dict(batch=1024, rows=2_000_000)}


def test_pack_keys_only_and_sentinel():
    # out-of-range indices form the sentinel key: slot -1, sent nowhere
    cfg = P.custom_cfg([50, 60], B=4, opt="sgd")
    keys = [np.array([1, 2, 50, 3]), np.array([-1, 5, 59, 60])]
    batch = W.make_batch_from_lengths([np.ones(4, int)] * 2, keys, 4, index_dtype=np.int64)
    u = np.array([1, 2, 3, 50 + 5, 50 + 59, 110])            # 110 = total rows = the sentinel
    P.say("pack sentinel")
    for grad in (False, True):
        tabs, *_ = _run_pack(cfg, batch, np.ones((4, 32), np.float32),
                             [(O.SHARD_ROW_CYCLIC, 1), (O.SHARD_TABLE, 0)], 2, unique_ref=u, grad=grad)
        with pytest.raises(Exception):
            tabs.check_device_error()                         # the bounds flag of the bad indices
        tabs.close()


def test_pack_empty_batch():
    cfg = P.custom_cfg([10, 20], B=5)
    batch = W.make_batch_from_lengths([np.zeros(5, int)] * 2, [np.zeros(0, int)] * 2, 5)
    P.say("pack empty")
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, np.ones((5, 32), np.float32))
    bufs = tabs.backward_buffers(0, 5, with_grad=False)
    tabs.backward(idx, off, 5, "sum", dy, bufs)
    tabs.set_shard_map([(O.SHARD_TABLE, 1), (O.SHARD_ROW_BLOCK, 0)], 3)
    pb = tabs.pack_buffers(0, 3, with_grad=False)
    pb["send_offsets"].fill_(-7)
    tabs.pack(bufs, pb)
    torch.cuda.synchronize()
    assert pb["send_offsets"].cpu().tolist() == [0, 0, 0, 0]
    tabs.close()


def test_update_after_pack_is_unchanged():
    # the pack uses only the sort scratch of the workspace: the fused update
    # that follows it writes the same bits as one with no pack in between
    cfg = W.make_config(2, batch=2048)
    batch = W.make_batch(cfg, k=3)
    dY = W.make_dy(cfg, k=3)
    P.say("update after pack cfg2")
    u, _, _ = P.oracle_dedup(cfg, batch)
    results = []
    for do_pack in (False, True):
        tabs = P.make_tables(cfg)
        idx, off, dy = P.to_dev(batch, dY)
        bufs = tabs.backward_buffers(batch.N, cfg.batch, with_grad=False)
        tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs)
        if do_pack:
            tabs.set_shard_map(_rules(lambda t: t % 3, cfg.T, 8), 8)
            pb = tabs.pack_buffers(batch.N, 8, with_grad=True)
            tabs.pack(bufs, pb, dY=dy)
        tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs, dY=dy)
        torch.cuda.synchronize()
        results.append(P.read_rows(tabs, cfg, u))
        tabs.close()
    assert np.array_equal(results[0][0].view(np.uint32), results[1][0].view(np.uint32))
    assert np.array_equal(results[0][1].view(np.uint32), results[1][1].view(np.uint32))


@pytest.mark.slow
def test_pack_full_size():
    # the 26 x 4M x 128 workload at batch 65536: 636 k unique keys routed to 64
    # shards, every key, offset and slot checked, the RB gradients bit-equal
    # to the unique-order reduction
    cfg = W.make_config(3)
    batch = W.make_batch(cfg, k=1)
    dY = W.make_dy(cfg, k=1)
    rules = _rules(lambda t: t % 3, cfg.T, 64)
    P.say("pack full cfg3 N", batch.N)
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, dY)
    bufs = tabs.backward_buffers(batch.N, cfg.batch, with_grad=True)
    tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs)
    tabs.set_shard_map(rules, 64)
    pb = tabs.pack_buffers(batch.N, 64, with_grad=True)
    tabs.pack(bufs, pb, dY=dy)
    torch.cuda.synchronize()
    u, _, _ = P.oracle_dedup(cfg, batch)
    U = int(bufs["num_unique"].item())
    assert U == len(u)
    ok, ooff, oslot, _ = O.pack_by_shard(u, cfg.row_offset(), rules, 64)
    assert np.array_equal(pb["send_offsets"].cpu().numpy().astype(np.int64), ooff)
    assert np.array_equal(pb["send_keys"][:U].cpu().numpy().view(np.uint32).astype(np.int64), ok)
    assert np.array_equal(pb["slot_of_unique"][:U].cpu().numpy().astype(np.int64), oslot)
    sg = pb["send_grad"][:U]
    rg = bufs["reduced_grad"][:U]
    slot = torch.from_numpy(oslot).cuda()
    assert torch.equal(sg[slot].view(torch.int32), rg.view(torch.int32))
    tabs.close()
