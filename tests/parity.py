"""Shared machinery of the GPU parity tests: run one training step of the HIP
path through the C ABI and compare it with the CPU oracle on the same seeded
inputs.

Tolerances (derived from the arithmetic; relative tolerance 1e-5 for fp32 and
2e-2 for 16-bit storage):
  pooled output  |Y - Y_ref| <= 1e-5 * M,  M = the same pooling of |W| (the
                 recursive-summation bound (L-1) * 2^-24 * M stays below it for
                 L <= 100; every stored value is exact in fp32);
  reduced grad   |g - g_ref| <= 1e-5 * M_g, M_g = sum of |scale * dY| of the
                 segment;
  updated rows   the oracle's update is monotone in g, so the GPU value must
                 lie between the oracle's updates at g_ref -+ 1e-5 * M_g,
                 widened by rtol_w * (|w_old| + |dw_ref|) for the update's own
                 rounding (rtol_w = 1e-5 fp32, 2e-2 bf16/fp16 storage);
  integers       unique keys, counts, inverse: bit-exact;
  untouched rows bit-exact (never written).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from dlrm_sparse_embedding_amd import emb as E
from dlrm_sparse_embedding_amd import workloads as W

RTOL_SUM = 1e-5
RTOL_W = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}


def make_tables(cfg: W.Config, master: bool = False) -> E.EmbeddingTables:
    specs = [E.TableSpec(t.rows, t.dim, t.dtype, t.col_slices) for t in cfg.tables]
    tabs = E.EmbeddingTables(specs, with_state=cfg.opt == "adagrad", with_master=master)
    tabs.init_uniform(cfg.init_seed)
    return tabs


def oracle_tables(cfg: W.Config, batch: W.Batch, extra_rows=None):
    """TouchedRows per table covering the batch's rows (+ extra rows)."""
    out = []
    B = batch.B
    for t in range(cfg.T):
        rows = batch.indices[int(batch.offsets[t * B]):int(batch.offsets[(t + 1) * B])].astype(np.int64)
        rows = rows[(rows >= 0) & (rows < cfg.tables[t].rows)]
        if extra_rows is not None and extra_rows[t] is not None:
            rows = np.concatenate([rows, np.asarray(extra_rows[t], np.int64)])
        out.append(O.TouchedRows(cfg.init_seed, t, cfg.dim, cfg.dtype, rows))
    return out


class _Abs:
    def __init__(self, tabs):
        self.tabs = tabs

    def __getitem__(self, t):
        tt = self.tabs[t]

        class _V:
            def __getitem__(self, r):
                return np.abs(tt[r])
        return _V()


def check_forward(Y_gpu: np.ndarray, cfg, batch, otabs, bags=None, num_rows=None):
    """Element-wise (or on sampled bags) forward check. num_rows: rows per
    table when some lookups name no row (they add nothing and count in L)."""
    if bags is None:
        ref = O.pooled_forward(otabs, batch.indices, batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool,
                               num_rows=num_rows)
        mag = O.pooled_forward(_Abs(otabs), batch.indices, batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool,
                               num_rows=num_rows)
        got = Y_gpu
    else:
        # sampled bags: build a sub-batch holding only them (sample b -> row j)
        sub = sub_batch(batch, cfg, bags)
        ref = O.pooled_forward(otabs, sub.indices, sub.offsets, sub.T, sub.B, cfg.dim, cfg.pool)
        mag = O.pooled_forward(_Abs(otabs), sub.indices, sub.offsets, sub.T, sub.B, cfg.dim, cfg.pool)
        got = Y_gpu
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bound = RTOL_SUM * mag.astype(np.float64)
    bad = err > bound
    assert not bad.any(), (f"forward: {int(bad.sum())} of {bad.size} elements off; worst "
                           f"err {err[bad].max():.3e} bound {bound[bad][np.argmax(err[bad])]:.3e}")
    return ref


def sub_batch(batch: W.Batch, cfg, samples: np.ndarray) -> W.Batch:
    """The bags of the given samples (all tables), as a batch of len(samples)."""
    B = cfg.batch
    lens, keys = [], []
    for t in range(cfg.T):
        bag = t * B + samples
        s = batch.offsets[bag].astype(np.int64)
        e = batch.offsets[bag + 1].astype(np.int64)
        lens.append(e - s)
        keys.append(np.concatenate([batch.indices[a:b] for a, b in zip(s, e)]) if len(s) else np.zeros(0, np.int64))
    return W.make_batch_from_lengths(lens, keys, len(samples), index_dtype=np.int64)


def to_dev(batch: W.Batch, dY: np.ndarray | None):
    idx = torch.from_numpy(batch.indices).cuda()
    off = torch.from_numpy(batch.offsets).cuda()
    dy = torch.from_numpy(dY).cuda() if dY is not None else None
    return idx, off, dy


def oracle_dedup(cfg, batch):
    ro = cfg.row_offset()
    g = O.global_keys(batch.indices, batch.offsets, ro, cfg.T, cfg.batch)
    return O.dedup(g)


def check_dedup(bufs, u, c, inv):
    U = int(bufs["num_unique"].item())
    assert U == len(u), (U, len(u))
    uk = bufs["unique_keys"][:U].cpu().numpy().view(np.uint32).astype(np.int64)
    assert np.array_equal(uk, u), "unique keys differ"
    assert np.array_equal(bufs["counts"][:U].cpu().numpy().astype(np.int64), c), "counts differ"
    N = len(inv)
    assert np.array_equal(bufs["inverse"][:N].cpu().numpy().astype(np.int64), inv), "inverse differs"
    return U


def grad_bounds(cfg, batch, dY, inv, U, select=None):
    g = O.reduced_grad(dY, batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool, inv, U, select=select)
    m = O.reduced_grad(np.abs(dY), batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool, inv, U, select=select)
    return g, m


def check_grad(g_gpu, g_ref, m_ref):
    err = np.abs(g_gpu.astype(np.float64) - g_ref.astype(np.float64))
    bound = RTOL_SUM * m_ref.astype(np.float64)
    bad = err > bound
    assert not bad.any(), f"reduced grad: {int(bad.sum())} elements off, worst {err.max():.3e}"


def check_update(cfg, w_gpu, G_gpu, w_old, G_old, g_ref, m_ref, wdtype=None):
    """w_gpu/G_gpu: device results (fp32 view of stored values) for the
    checked rows; w_old: stored values before the step. wdtype: the type the
    checked weights are kept in (default the storage type; "f32" for an fp32
    master)."""
    delta = RTOL_SUM * m_ref.astype(np.float32)
    g_lo = (g_ref - delta).astype(np.float32)
    g_hi = (g_ref + delta).astype(np.float32)
    if cfg.opt == "sgd":
        wr = O.sgd_step(w_old, g_ref, cfg.lr)
        wa, wb = O.sgd_step(w_old, g_lo, cfg.lr), O.sgd_step(w_old, g_hi, cfg.lr)
    else:
        wr, Gr = O.adagrad_step(w_old, G_old, g_ref, cfg.lr, cfg.eps)
        wa, Ga = O.adagrad_step(w_old, G_old, g_lo, cfg.lr, cfg.eps)
        wb, Gb = O.adagrad_step(w_old, G_old, g_hi, cfg.lr, cfg.eps)
    tol = RTOL_W[wdtype or cfg.dtype] * (np.abs(w_old).astype(np.float64) + np.abs(wr.astype(np.float64) - w_old))
    lo = np.minimum(wa, wb).astype(np.float64) - tol
    hi = np.maximum(wa, wb).astype(np.float64) + tol
    wg = w_gpu.astype(np.float64)
    bad = (wg < lo) | (wg > hi)
    assert not bad.any(), (f"updated rows: {int(bad.sum())} of {bad.size} off; e.g. got {wg[bad][:3]} "
                           f"want [{lo[bad][:3]}, {hi[bad][:3]}]")
    if cfg.opt == "adagrad":
        # G' = G + g^2 is monotone in |g|
        ga = np.minimum(np.abs(g_lo), np.abs(g_hi))
        ga = np.where(np.sign(g_lo) != np.sign(g_hi), 0.0, ga).astype(np.float32)
        gb = np.maximum(np.abs(g_lo), np.abs(g_hi)).astype(np.float32)
        Glo = (G_old + ga * ga).astype(np.float64)
        Ghi = (G_old + gb * gb).astype(np.float64)
        tG = 1e-5 * np.abs(Ghi)
        Gg = G_gpu.astype(np.float64)
        badG = (Gg < Glo - tG) | (Gg > Ghi + tG)
        assert not badG.any(), f"Adagrad state: {int(badG.sum())} elements off"


def read_rows(tabs: E.EmbeddingTables, cfg, keys: np.ndarray):
    """Stored values (as fp32) and state of global keys, grouped by table."""
    ro = cfg.row_offset()
    t_of = np.searchsorted(ro, keys, side="right") - 1
    w = np.zeros((len(keys), cfg.dim), np.float32)
    G = np.zeros((len(keys), cfg.dim), np.float32) if cfg.opt == "adagrad" else None
    for t in np.unique(t_of):
        sel = np.nonzero(t_of == t)[0]
        rows = keys[sel] - ro[t]
        w[sel] = tabs.logical_rows(int(t), rows).float().cpu().numpy()
        if G is not None:
            G[sel] = tabs.logical_state(int(t), rows).cpu().numpy()
    return w, G


def read_master(tabs: E.EmbeddingTables, cfg, keys: np.ndarray):
    """fp32 master rows of global keys."""
    ro = cfg.row_offset()
    t_of = np.searchsorted(ro, keys, side="right") - 1
    m = np.zeros((len(keys), cfg.dim), np.float32)
    for t in np.unique(t_of):
        sel = np.nonzero(t_of == t)[0]
        m[sel] = tabs.logical_master(int(t), keys[sel] - ro[t]).cpu().numpy()
    return m


def stored_init(cfg, keys: np.ndarray, rounded: bool = True):
    """Initial values of global keys: as stored (rounded to the storage
    type), or the fp32 values an fp32 master starts from."""
    ro = cfg.row_offset()
    t_of = np.searchsorted(ro, keys, side="right") - 1
    w = np.zeros((len(keys), cfg.dim), np.float32)
    for t in np.unique(t_of):
        sel = np.nonzero(t_of == t)[0]
        v = O.init_values(cfg.init_seed, int(t), keys[sel] - ro[t], cfg.dim)
        w[sel] = O.to_storage(v, cfg.dtype) if rounded else v
    return w


def update_interval(cfg, w_lo, w_hi, G_lo, G_hi, g_ref, m_ref, wdtype=None):
    """Propagates an interval of (w, G) through one oracle step with the
    gradient known to within +-1e-5 * m_ref. The step is monotone in each of
    w, G and g separately (increasing in w, decreasing in g, and in G
    increasing or decreasing with the sign of g), so its extremes over the box
    are at its corners; the interval is widened by the step's own rounding.
    Used to chain several steps from oracle values only."""
    delta = RTOL_SUM * m_ref.astype(np.float32)
    gs = [(g_ref - delta).astype(np.float32), (g_ref + delta).astype(np.float32)]
    rt = RTOL_W[wdtype or cfg.dtype]
    ws = []
    for w in (w_lo, w_hi):
        for g in gs:
            if cfg.opt == "sgd":
                ws.append(O.sgd_step(w, g, cfg.lr))
            else:
                for G in (G_lo, G_hi):
                    ws.append(O.adagrad_step(w, G, g, cfg.lr, cfg.eps)[0])
    ws = np.stack(ws).astype(np.float64)
    span = np.abs(ws - np.stack([w_lo] * len(ws)).astype(np.float64)).max(axis=0)
    tol = rt * (np.abs(w_lo).astype(np.float64) + span)
    lo, hi = ws.min(axis=0) - tol, ws.max(axis=0) + tol
    if cfg.opt == "sgd":
        return lo, hi, G_lo, G_hi
    # G' = G + g*g rises with G but not with g: over a gradient band that
    # holds 0 its least g*g is 0, else that of the band's end nearer 0
    g_lo, g_hi = gs
    sq_lo = np.where((g_lo <= 0) & (g_hi >= 0), np.float32(0), np.minimum(g_lo * g_lo, g_hi * g_hi))
    sq_hi = np.maximum(g_lo * g_lo, g_hi * g_hi)
    Gl = (np.asarray(G_lo, np.float32) + sq_lo.astype(np.float32)).astype(np.float64)
    Gh = (np.asarray(G_hi, np.float32) + sq_hi.astype(np.float32)).astype(np.float64)
    tG = 1e-5 * np.abs(Gh)
    return lo, hi, Gl - tG, Gh + tG


def check_interval(name, got, lo, hi):
    g = np.asarray(got, np.float64)
    bad = (g < lo) | (g > hi)
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} off; e.g. got {g[bad][:3]} "
                           f"want [{lo[bad][:3]}, {hi[bad][:3]}]")


def run_step(cfg, batch, dY, path="fused", sample_bags=None, sample_keys=None, sample_untouched=2000,
             seed=0, tabs=None, master=False):
    """Forward + backward + update on the GPU; every check against the oracle.
    sample_bags / sample_keys: None = check everything; else the number of
    sampled samples / unique keys to check. master: the tables carry fp32
    master weights (the update steps the master; the stored copy must be its
    RNE cast, bit for bit)."""
    rng = np.random.default_rng(seed)
    own = tabs is None
    if own:
        tabs = make_tables(cfg, master=master)
    idx, off, dy = to_dev(batch, dY)
    B, N = cfg.batch, batch.N
    # ---- forward
    Y = tabs.forward(idx, off, B, cfg.pool)
    torch.cuda.synchronize()
    tabs.check_device_error()
    if sample_bags is None:
        otabs = oracle_tables(cfg, batch)
        check_forward(Y.cpu().numpy(), cfg, batch, otabs)
    else:
        samples = np.sort(rng.choice(B, min(sample_bags, B), replace=False))
        sub = sub_batch(batch, cfg, samples)
        otabs = oracle_tables(cfg, sub)
        check_forward(Y[torch.from_numpy(samples).cuda()].cpu().numpy(), cfg, batch, otabs, bags=samples)
    del Y
    # ---- backward (dedup [+ materialised gradient])
    bufs = tabs.backward_buffers(N, B, with_grad=(path == "materialized"))
    tabs.backward(idx, off, B, cfg.pool, dy, bufs)
    torch.cuda.synchronize()
    u, c, inv = oracle_dedup(cfg, batch)
    U = check_dedup(bufs, u, c, inv)
    if sample_keys is None or sample_keys >= U:
        sel = np.arange(U)
    else:
        sel = np.sort(np.concatenate([rng.choice(U, sample_keys, replace=False),
                                      np.argsort(-c)[:16]]))   # always the hottest keys
        sel = np.unique(sel)
    g_ref, m_ref = grad_bounds(cfg, batch, dY, inv, U, select=sel if len(sel) < U else None)
    if path == "materialized":
        g_gpu = bufs["reduced_grad"][torch.from_numpy(sel).cuda()].cpu().numpy()
        check_grad(g_gpu, g_ref, m_ref)
    # ---- update
    keys = u[sel]
    w_old = stored_init(cfg, keys, rounded=not master)
    G_old = np.zeros_like(w_old) if cfg.opt == "adagrad" else None
    tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs, dY=dy)
    torch.cuda.synchronize()
    tabs.check_device_error()
    w_new, G_new = read_rows(tabs, cfg, keys)
    if master:
        m_new = read_master(tabs, cfg, keys)
        check_update(cfg, m_new, G_new, w_old, G_old, g_ref, m_ref, wdtype="f32")
        # the stored copy is the RNE cast of the device's own master: one
        # rounding decision, taken in the same precision on both sides
        assert np.array_equal(w_new.view(np.uint32), O.to_storage(m_new, cfg.dtype).view(np.uint32)), \
            "stored copy is not the RNE cast of the master"
    else:
        check_update(cfg, w_new, G_new, w_old, G_old, g_ref, m_ref)
    # ---- untouched rows stay bit-identical
    if sample_untouched:
        tot = cfg.total_rows
        cand = np.unique(rng.integers(0, tot, sample_untouched * 2))
        cand = cand[~np.isin(cand, u)][:sample_untouched]
        if len(cand):
            w_u, G_u = read_rows(tabs, cfg, cand)
            assert np.array_equal(w_u.view(np.uint32), stored_init(cfg, cand).view(np.uint32)), "untouched row changed"
            if master:
                assert np.array_equal(read_master(tabs, cfg, cand).view(np.uint32),
                                      stored_init(cfg, cand, rounded=False).view(np.uint32)), "untouched master changed"
            if G_u is not None:
                assert np.all(G_u == 0), "untouched state changed"
    result = dict(U=U, keys=keys, w_new=w_new, G_new=G_new, bufs=bufs)
    if own:
        tabs.close()
    return result


def say(*a):
    print("[case]", *a, flush=True)


def custom_cfg(rows, dim=16, dtype="f32", slices=1, B=8, pool="sum", opt="adagrad"):
    tabs = tuple(W.TableSpec(r, dim, dtype, slices) for r in rows)
    return W.Config(99, "custom", tabs, B, pool, opt, 0.05, 1e-8, tuple(1 for _ in rows), None, init_seed=99)
