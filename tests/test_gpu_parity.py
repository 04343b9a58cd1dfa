"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Run on an MI355X:  python -u -m pytest tests -m gpu -x -v --timeout 300
Every case prints its name, seed and shape before it touches the GPU.
"""
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


def _say(*a):
    print("[case]", *a, flush=True)


# ---------------------------------------------------------------------------
# table contents: device counter hash == oracle counter hash, bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,dim,slices", [("f32", 16, 1), ("f32", 128, 1), ("bf16", 128, 1),
                                              ("f16", 128, 4), ("f16", 64, 2), ("bf16", 8, 1)])
def test_init_bit_exact(dtype, dim, slices):
    _say("init", dtype, dim, slices)
    specs = [E.TableSpec(1000, dim, dtype, slices), E.TableSpec(37, dim, dtype, slices)]
    tabs = E.EmbeddingTables(specs, with_state=True)
    tabs.init_uniform(12345)
    torch.cuda.synchronize()
    for t, sp in enumerate(specs):
        rows = np.arange(sp.rows)
        got = tabs.logical_rows(t, rows).float().cpu().numpy()
        ref = O.to_storage(O.init_values(12345, t, rows, dim), dtype)
        bad = got.view(np.uint32) != ref.view(np.uint32)
        if bad.any():
            r, c = np.nonzero(bad)
            raise AssertionError(f"table {t}: {int(bad.sum())} of {bad.size} differ; first (row, col, got, ref): "
                                 f"{[(int(a), int(b), float(got[a, b]), float(ref[a, b])) for a, b in zip(r[:6], c[:6])]}")
        assert torch.all(tabs.logical_state(t, rows) == 0)
    tabs.close()


# ---------------------------------------------------------------------------
# the five configurations, oracle-sized: every element checked
# ---------------------------------------------------------------------------

REDUCED = {1: dict(), 2: dict(batch=2048), 3: dict(batch=1024), 4: dict(batch=48), 5: dict(batch=1024)}


@pytest.mark.parametrize("path", ["fused", "materialized"])
@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_config_reduced(cfg_id, path):
    cfg = W.make_config(cfg_id, **REDUCED[cfg_id])
    batch = W.make_batch(cfg)
    dY = W.make_dy(cfg)
    _say(f"cfg{cfg_id} reduced B={cfg.batch} N={batch.N} path={path}")
    r = P.run_step(cfg, batch, dY, path=path)
    assert r["U"] > 0


# ---------------------------------------------------------------------------
# full sizes, launch configuration of the benchmark, sampled outputs
# ---------------------------------------------------------------------------

@pytest.mark.slow
@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5])
def test_config_full_sampled(cfg_id):
    cfg = W.make_config(cfg_id)
    batch = W.make_batch(cfg)
    dY = W.make_dy(cfg)
    _say(f"cfg{cfg_id} full B={cfg.batch} N={batch.N}")
    P.run_step(cfg, batch, dY, path="fused", sample_bags=512, sample_keys=3000)


@pytest.mark.slow
def test_master_weights_full_sampled():
    # the 100 x 1M x 128 bf16 workload (mean pooling, SGD) with fp32 masters at
    # its full batch: 25.6 GB of bf16 rows + 51.2 GB of masters
    cfg = W.make_config(4)
    batch = W.make_batch(cfg)
    dY = W.make_dy(cfg)
    _say(f"cfg4 full with masters N={batch.N}")
    P.run_step(cfg, batch, dY, path="fused", sample_bags=256, sample_keys=3000, master=True)


# ---------------------------------------------------------------------------
# exactness: integer upstream gradients make every fp32 sum exact, so the
# fused sparse update must equal the oracle bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg_id,opt", [(1, "sgd"), (1, "adagrad"), (2, "adagrad"), (2, "sgd")])
def test_integer_grad_bit_exact(cfg_id, opt):
    from dataclasses import replace
    cfg = replace(W.make_config(cfg_id, **REDUCED[cfg_id]), opt=opt, eps=1e-8)
    batch = W.make_batch(cfg)
    dY = W.make_int_dy(cfg)
    _say(f"int-grad cfg{cfg_id} {opt} N={batch.N}")
    r = P.run_step(cfg, batch, dY, path="fused")
    u, c, inv = P.oracle_dedup(cfg, batch)
    g = O.reduced_grad(dY, batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool, inv, len(u))
    w_old = P.stored_init(cfg, u)
    G_old = np.zeros_like(w_old) if opt == "adagrad" else None
    w_ref, G_ref = O.update_rows(w_old, G_old, g, opt, cfg.lr, cfg.eps, cfg.dtype)
    assert np.array_equal(r["w_new"].view(np.uint32), w_ref.view(np.uint32))
    if opt == "adagrad":
        assert np.array_equal(r["G_new"].view(np.uint32), G_ref.view(np.uint32))


# 16-bit storage: integer dY, sum pooling and lr = 2^-7 make the fp32 step
# exact up to its own IEEE roundings (SGD: one subtraction; Adagrad: sqrt,
# add, divide, subtract), so the stored bf16 / fp16 bits -- the
# round-to-nearest-even write-back, or the master and its RNE copy -- must
# equal the oracle's bit for bit. A truncating write-back differs from RNE in
# about half the elements and fails here; the 2e-2 band cannot tell them apart.
LOWP_EXACT = [(4, "sgd", False), (4, "sgd", True), (4, "adagrad", False),
              (5, "sgd", False), (5, "adagrad", False), (5, "adagrad", True)]


@pytest.mark.parametrize("cfg_id,opt,master", LOWP_EXACT)
def test_integer_grad_bit_exact_low_precision(cfg_id, opt, master):
    from dataclasses import replace
    base = W.make_config(cfg_id, rows=2_000_000, **REDUCED[cfg_id])
    if opt == "adagrad" and base.opt != "adagrad":
        # Adagrad on a bf16 table that carries no state in its own workload
        base = replace(base, opt="adagrad")
    cfg = replace(base, pool="sum", opt=opt, lr=2.0 ** -7, eps=1e-8)
    batch = W.make_batch(cfg)
    dY = W.make_int_dy(cfg)
    _say(f"int-grad {cfg.dtype} cfg{cfg_id} {opt} master={master} N={batch.N}")
    tabs = P.make_tables(cfg, master=master)
    r = P.run_step(cfg, batch, dY, path="fused", tabs=tabs, sample_untouched=200, master=master)
    u, c, inv = P.oracle_dedup(cfg, batch)
    g = O.reduced_grad(dY, batch.offsets, cfg.T, cfg.batch, cfg.dim, cfg.pool, inv, len(u))
    assert np.all(np.abs(g) < 2 ** 24) and np.array_equal(g, np.round(g))   # every sum exact
    G_old = np.zeros((len(u), cfg.dim), np.float32) if opt == "adagrad" else None
    if master:
        m_old = P.stored_init(cfg, u, rounded=False)
        m_ref, w_ref, G_ref = O.update_rows_master(m_old, G_old, g, opt, cfg.lr, cfg.eps, cfg.dtype)
        m_new = P.read_master(tabs, cfg, u)
        assert np.array_equal(m_new.view(np.uint32), m_ref.view(np.uint32)), "master differs"
    else:
        w_old = P.stored_init(cfg, u)
        w_ref, G_ref = O.update_rows(w_old, G_old, g, opt, cfg.lr, cfg.eps, cfg.dtype)
    moved = np.mean(w_ref != P.stored_init(cfg, u))
    assert moved > 0.5, moved                      # the step is visible in the stored type
    bad = r["w_new"].view(np.uint32) != w_ref.view(np.uint32)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} stored elements differ from the oracle's RNE"
    if opt == "adagrad":
        assert np.array_equal(r["G_new"].view(np.uint32), G_ref.view(np.uint32))
    tabs.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_out_of_range_mean_matches_oracle(dtype):
    # mean pooling over bags that hold indices outside their table: such a
    # lookup adds nothing and still counts in its bag's length, in the forward
    # and in the 1/L of its bag's other lookups in the backward (the oracle's
    # definition); its own key is the never-applied sentinel
    rng = np.random.default_rng(17)
    rows = [40, 900, 7]
    cfg = _custom_cfg(rows, dim=32, dtype=dtype, B=300, pool="mean", opt="sgd")
    lens = [rng.integers(0, 6, cfg.batch) for _ in rows]
    keys = []
    for t, r in enumerate(rows):
        k = rng.integers(0, r, int(lens[t].sum()))
        bad = rng.random(len(k)) < 0.3
        k[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1 - rng.integers(0, 5, int(bad.sum())),
                          r + rng.integers(0, 5, int(bad.sum())))
        keys.append(k)
    batch = W.make_batch_from_lengths(lens, keys, cfg.batch, index_dtype=np.int64)
    dY = rng.standard_normal((cfg.batch, cfg.T * cfg.dim)).astype(np.float32)
    _say("out-of-range mean", dtype, batch.N)
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, dY)
    Y = tabs.forward(idx, off, cfg.batch, "mean")
    torch.cuda.synchronize()
    with pytest.raises(E.EmbError) as ei:
        tabs.check_device_error()
    assert ei.value.code == E.EMB_E_BOUNDS
    otabs = P.oracle_tables(cfg, batch)
    P.check_forward(Y.cpu().numpy(), cfg, batch, otabs, num_rows=rows)
    bufs = tabs.backward_buffers(batch.N, cfg.batch, with_grad=True)
    tabs.backward(idx, off, cfg.batch, "mean", dy, bufs)
    torch.cuda.synchronize()
    # in-range keys, counts and inverse as the oracle's dedup of the lookups
    # that found a row; row-less lookups point at the sentinel key
    ro = cfg.row_offset()
    t_of = np.repeat(np.arange(cfg.T), np.diff(batch.offsets[::cfg.batch].astype(np.int64)))
    found = (batch.indices >= 0) & (batch.indices < np.asarray(rows)[t_of])
    g_all = ro[t_of] + batch.indices
    u, c, inv_f = O.dedup(g_all[found])
    U = int(bufs["num_unique"].item())
    uk = bufs["unique_keys"][:U].cpu().numpy().view(np.uint32).astype(np.int64)
    cg = bufs["counts"][:U].cpu().numpy().astype(np.int64)
    inv_g = bufs["inverse"][:batch.N].cpu().numpy().astype(np.int64)
    valid = uk < cfg.total_rows
    assert np.array_equal(uk[valid], u) and np.array_equal(cg[valid], c)
    assert np.array_equal(uk[inv_g[found]], g_all[found])
    assert np.all(uk[inv_g[~found]] == cfg.total_rows)
    inv = np.full(batch.N, -1, np.int64)
    inv[found] = inv_f
    g_ref = O.reduced_grad(dY, batch.offsets, cfg.T, cfg.batch, cfg.dim, "mean", inv, len(u))
    m_ref = O.reduced_grad(np.abs(dY), batch.offsets, cfg.T, cfg.batch, cfg.dim, "mean", inv, len(u))
    slot = np.nonzero(valid)[0]
    P.check_grad(bufs["reduced_grad"][torch.from_numpy(slot).cuda()].cpu().numpy(), g_ref, m_ref)
    tabs.update("sgd", cfg.lr, 0.0, bufs, dY=dy)
    torch.cuda.synchronize()
    with pytest.raises(E.EmbError):
        tabs.check_device_error()
    w_new, _ = P.read_rows(tabs, cfg, u)
    P.check_update(cfg, w_new, None, P.stored_init(cfg, u), None, g_ref, m_ref)
    # rows no lookup found are untouched
    rest = np.setdiff1d(np.arange(cfg.total_rows), u)
    w_rest, _ = P.read_rows(tabs, cfg, rest)
    assert np.array_equal(w_rest.view(np.uint32), P.stored_init(cfg, rest).view(np.uint32))
    tabs.close()


def test_fused_equals_materialized_and_reruns_bit_identical():
    cfg = W.make_config(2, batch=4096)
    batch = W.make_batch(cfg, k=3)
    dY = W.make_dy(cfg, k=3)
    _say("determinism cfg2 B=4096")
    res = []
    for path in ("fused", "materialized", "fused"):
        res.append(P.run_step(cfg, batch, dY, path=path, sample_untouched=0))
    for r in res[1:]:
        assert np.array_equal(r["w_new"].view(np.uint32), res[0]["w_new"].view(np.uint32))
        assert np.array_equal(r["G_new"].view(np.uint32), res[0]["G_new"].view(np.uint32))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _custom_cfg(rows, dim=16, dtype="f32", slices=1, B=8, pool="sum", opt="adagrad"):
    tabs = tuple(W.TableSpec(r, dim, dtype, slices) for r in rows)
    return W.Config(99, "custom", tabs, B, pool, opt, 0.05, 1e-8, tuple(1 for _ in rows), None, init_seed=99)


@pytest.mark.parametrize("pool", ["sum", "mean"])
@pytest.mark.parametrize("itype", [np.int32, np.int64])
def test_empty_and_ragged_bags(pool, itype):
    rng = np.random.default_rng(11)
    cfg = _custom_cfg([1, 7, 300, 5000], dim=32, B=333, pool=pool)
    lens = [rng.integers(0, 6, cfg.batch) * (rng.random(cfg.batch) < 0.7) for _ in range(cfg.T)]
    lens[1][:] = 0                                   # a table with only empty bags
    keys = [rng.integers(0, cfg.tables[t].rows, int(lens[t].sum())) for t in range(cfg.T)]
    batch = W.make_batch_from_lengths(lens, keys, cfg.batch, index_dtype=itype)
    dY = np.random.default_rng(1).standard_normal((cfg.batch, cfg.T * cfg.dim)).astype(np.float32)
    _say("ragged", pool, itype.__name__, batch.N)
    P.run_step(cfg, batch, dY, path="materialized")
    P.run_step(cfg, batch, dY, path="fused")


def test_all_empty_batch():
    cfg = _custom_cfg([10, 20], B=17)
    batch = W.make_batch_from_lengths([np.zeros(17, int)] * 2, [np.zeros(0, int)] * 2, 17)
    _say("all-empty")
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, np.ones((17, 32), np.float32))
    Y = tabs.forward(idx, off, 17, "mean")
    bufs = tabs.backward_buffers(0, 17, with_grad=True)
    tabs.backward(idx, off, 17, "mean", dy, bufs)
    tabs.update("adagrad", 0.1, 1e-8, bufs, dY=dy)
    torch.cuda.synchronize()
    assert torch.all(Y == 0) and int(bufs["num_unique"].item()) == 0
    tabs.close()


@pytest.mark.parametrize("n,dim,dtype", [(50000, 128, "f32"), (20000, 64, "bf16"), (1000, 128, "f16")])
def test_single_hot_key_long_segment(n, dim, dtype):
    # one key looked up n times (one segment of length n, split over many
    # chunks and combined), next to a few keys of other lengths
    rng = np.random.default_rng(5)
    cfg = _custom_cfg([100, 1000], dim=dim, dtype=dtype, B=n)
    k0 = np.full(n, 42)
    k1 = rng.integers(0, 1000, n)
    k1[: n // 2] = 7                                   # second long segment, in table 1
    batch = W.make_batch_from_lengths([np.ones(n, int), np.ones(n, int)], [k0, k1], n)
    dY = rng.standard_normal((n, 2 * dim)).astype(np.float32)
    _say("hot-key", n, dim, dtype)
    for path in ("materialized", "fused"):
        P.run_step(cfg, batch, dY, path=path)


def test_segments_on_chunk_boundaries():
    # segment lengths straddling the 128-position chunk grid exactly
    lens_seq = [128, 128, 1, 127, 129, 256, 255, 257, 1, 1, 384, 2]
    keys = np.concatenate([np.full(L, i * 3) for i, L in enumerate(lens_seq)])
    rng = np.random.default_rng(2)
    rng.shuffle(keys)
    n = len(keys)
    cfg = _custom_cfg([64], dim=16, B=n, opt="sgd")
    batch = W.make_batch_from_lengths([np.ones(n, int)], [keys], n)
    dY = rng.standard_normal((n, 16)).astype(np.float32)
    _say("chunk-boundaries", n)
    for path in ("materialized", "fused"):
        P.run_step(cfg, batch, dY, path=path)


@pytest.mark.parametrize("dim", [16, 128])
def test_out_of_range_index_flagged_not_applied(dim):
    # 128 columns: the reduce's waves read their chunk descriptors in pairs,
    # and the sentinel segment's chunk takes its own path through that loop
    cfg = _custom_cfg([50, 60], dim=dim, B=4, opt="sgd")
    keys = [np.array([1, 2, 50, 3]), np.array([-1, 5, 59, 60])]   # 50, -1, 60 out of range
    batch = W.make_batch_from_lengths([np.ones(4, int)] * 2, keys, 4, index_dtype=np.int64)
    _say("out-of-range", dim)
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, np.ones((4, 2 * dim), np.float32))
    Y = tabs.forward(idx, off, 4, "sum")
    with pytest.raises(E.EmbError) as ei:
        tabs.check_device_error()
    assert ei.value.code == E.EMB_E_BOUNDS
    y = Y.cpu().numpy()
    assert np.all(y[2, :dim] == 0) and np.all(y[0, dim:] == 0) and np.all(y[3, dim:] == 0)
    bufs = tabs.backward_buffers(8, 4, with_grad=False)
    tabs.backward(idx, off, 4, "sum", dy, bufs)
    tabs.update("sgd", 0.5, 0.0, bufs, dY=dy)
    with pytest.raises(E.EmbError):
        tabs.check_device_error()
    U = int(bufs["num_unique"].item())
    uk = bufs["unique_keys"][:U].cpu().numpy().view(np.uint32)
    assert uk[-1] == cfg.total_rows          # the sentinel segment sorts last
    tabs.check_device_error()                # flag was cleared
    # valid rows were updated, the rest of both tables is untouched
    w, _ = P.read_rows(tabs, cfg, np.arange(cfg.total_rows))
    init = P.stored_init(cfg, np.arange(cfg.total_rows))
    touched = np.array([1, 2, 3, 50 + 5, 50 + 59])
    changed = np.nonzero(np.any(w != init, axis=1))[0]
    assert np.array_equal(changed, touched)
    tabs.close()


# tables sorted globally (one radix pass over the keys) and tables sorted per
# table on their row bits (the segments come from the table starts in the
# offsets, so malformed offsets reach the sort's segment map)
OFFSET_TABLES = {"global": [50, 60], "per_table": [1000, 700, 1023, 10, 500, 999]}


@pytest.mark.parametrize("tables", sorted(OFFSET_TABLES))
@pytest.mark.parametrize("case", ["decreasing", "short_end", "long_end", "nonzero_start", "table_start_past_next"])
def test_malformed_offsets_flagged(case, tables):
    # offsets that break the CSR contract: the backward's key build reports
    # EMB_E_INVAL through the device flag; every kernel clamps offsets into
    # [0, N], so the whole step still runs inside the caller's buffers
    rows = OFFSET_TABLES[tables]
    T = len(rows)
    cfg = _custom_cfg(rows, B=8, opt="sgd")
    rng = np.random.default_rng(11)
    lens = [rng.integers(0, 4, 8) for _ in rows]
    keys = [rng.integers(0, r, int(l.sum())) for r, l in zip(rows, lens)]
    batch = W.make_batch_from_lengths(lens, keys, 8)
    off = batch.offsets.copy()
    N = batch.N
    if case == "decreasing":
        off[5] = off[7] + 1
        off[6] = 0
    elif case == "short_end":
        off[-1] = N - 3
        off[-2] = min(off[-2], N - 3)
    elif case == "long_end":
        off[-1] = N + 5
    elif case == "nonzero_start":
        off[0] = 2
    else:  # table 1 starts past table 2's start (past the end with two tables)
        off[8] = off[16] + 1
    _say("malformed offsets", case, tables)
    tabs = P.make_tables(cfg)
    idx = torch.from_numpy(batch.indices).cuda()
    offd = torch.from_numpy(off).cuda()
    dy = torch.ones((8, T * 16), dtype=torch.float32, device="cuda")
    tabs.forward(idx, offd, 8, "mean")
    bufs = tabs.backward_buffers(N, 8, with_grad=False)
    tabs.backward(idx, offd, 8, "mean", dy, bufs)
    tabs.update("sgd", 0.5, 0.0, bufs, dY=dy)
    with pytest.raises(E.EmbError) as ei:
        tabs.check_device_error()
    if tables == "global" and case != "table_start_past_next":
        assert ei.value.code == E.EMB_E_INVAL
    else:
        # positions the broken offsets hand to another table's bags may also
        # hold rows outside that table, which is reported first
        assert ei.value.code in (E.EMB_E_INVAL, E.EMB_E_BOUNDS)
    tabs.check_device_error()                # flag was cleared
    tabs.close()


def _chained_steps(cfg, batches, dys, master=False):
    """Several training steps on one set of tables. The expected rows come
    from the oracle alone: each touched row's (w, G) is carried as an interval
    from step to step (update_interval), never from the device's results."""
    tabs = P.make_tables(cfg, master=master)
    box = {}   # key -> (w_lo, w_hi, G_lo, G_hi) from the oracle chain
    for batch, dY in zip(batches, dys):
        idx, off, dy = P.to_dev(batch, dY)
        bufs = tabs.backward_buffers(batch.N, cfg.batch, with_grad=False)
        tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs)
        tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs, dY=dy)
        torch.cuda.synchronize()
        u, c, inv = P.oracle_dedup(cfg, batch)
        g, m = P.grad_bounds(cfg, batch, dY, inv, len(u))
        w0 = P.stored_init(cfg, u, rounded=not master).astype(np.float64)
        w_lo, w_hi = w0.copy(), w0.copy()
        G_lo, G_hi = np.zeros_like(w0), np.zeros_like(w0)
        for j, k in enumerate(u.tolist()):
            if k in box:
                w_lo[j], w_hi[j], G_lo[j], G_hi[j] = box[k]
        f32 = lambda a: a.astype(np.float32)
        lo, hi, Glo, Ghi = P.update_interval(cfg, f32(w_lo), f32(w_hi), f32(G_lo), f32(G_hi), g, m,
                                             wdtype="f32" if master else None)
        w_new, G_new = P.read_rows(tabs, cfg, u)
        if master:
            m_new = P.read_master(tabs, cfg, u)
            P.check_interval("master", m_new, lo, hi)
            assert np.array_equal(w_new.view(np.uint32), O.to_storage(m_new, cfg.dtype).view(np.uint32))
        else:
            P.check_interval("weights", w_new, lo, hi)
        if cfg.opt == "adagrad":
            P.check_interval("state", G_new, Glo, Ghi)
        for j, k in enumerate(u.tolist()):
            box[k] = (lo[j], hi[j], Glo[j], Ghi[j])
    tabs.close()


def test_two_adagrad_steps():
    cfg = W.make_config(2, batch=3000)
    _say("two-steps cfg2")
    _chained_steps(cfg, [W.make_batch(cfg, k=0), W.make_batch(cfg, k=1)],
                   [W.make_dy(cfg, k=0), W.make_dy(cfg, k=1)])


@pytest.mark.parametrize("cfg_id,path", [(4, "fused"), (4, "materialized"), (5, "fused"), (5, "materialized")])
def test_master_weights_step(cfg_id, path):
    # bf16 (SGD, mean pooling) and fp16 (Adagrad, 4 column slices) tables with
    # fp32 masters: master within the fp32 band, stored copy = RNE(master)
    # the masters add 4 bytes per element: tables shrunk to 2M rows
    cfg = W.make_config(cfg_id, rows=2_000_000, **REDUCED[cfg_id])
    batch = W.make_batch(cfg, k=0)
    dY = W.make_dy(cfg, k=0)
    _say("master", cfg_id, path)
    P.run_step(cfg, batch, dY, path=path, master=True)


def test_master_weights_three_steps():
    # fp16 Adagrad with fp32 masters over three steps: the masters follow the
    # oracle's fp32 chain (a step taken from the rounded copy would leave it)
    cfg = W.make_config(5, batch=512, rows=2_000_000)
    _say("master three steps cfg5")
    _chained_steps(cfg, [W.make_batch(cfg, k=k) for k in range(3)], [W.make_dy(cfg, k=k) for k in range(3)],
                   master=True)


@pytest.mark.parametrize("cfg_id,ahead", [(2, 1), (5, 1), (2, 2), (5, 2)])
def test_pipelined_dedup_matches_serial(cfg_id, ahead):
    # four steps where the dedup of the batch `ahead` steps on runs on a side
    # stream, into its own workspace (ahead + 1 of them, so up to `ahead`
    # dedups are pending at once), while the current step's forward and
    # update run -- the pattern of bench.py's pipeline schedule -- against
    # four serial steps (one-hot tables; and the multi-hot column-sliced fp16
    # shard). Every backward must find its dedup done ahead and skip its own.
    cfg = W.make_config(2, batch=4096) if cfg_id == 2 else W.make_config(5, batch=4096, rows=2_000_000)
    K = 4
    batches = [W.make_batch(cfg, k=k) for k in range(K)]
    dys = [W.make_dy(cfg, k=k) for k in range(K)]
    u = np.unique(np.concatenate([P.oracle_dedup(cfg, b)[0] for b in batches]))
    _say("pipelined dedup cfg", cfg_id, "ahead", ahead)
    results = []
    for pipelined in (False, True):
        tabs = P.make_tables(cfg)
        E.emb_set_kernel_timing(tabs.ctx, True)
        nset = ahead + 1
        dev = [P.to_dev(b, d) for b, d in zip(batches, dys)]
        bufs = [tabs.backward_buffers(max(b.N for b in batches), cfg.batch, with_grad=False) for _ in range(nset)]
        main, side = torch.cuda.current_stream(), torch.cuda.Stream()
        free = [torch.cuda.Event() for _ in range(nset)]
        done = [torch.cuda.Event() for _ in range(nset)]
        for e in free:
            e.record(main)

        def dedup_ahead(i):
            side.wait_event(free[i % nset])
            with torch.cuda.stream(side):
                tabs.dedup(dev[i][0], dev[i][1], cfg.batch, cfg.pool, bufs[i % nset])
            done[i % nset].record(side)

        if pipelined:
            for i in range(ahead):
                dedup_ahead(i)
        for i in range(K):
            idx, off, dy = dev[i]
            tabs.forward(idx, off, cfg.batch, cfg.pool)
            if pipelined:
                main.wait_event(done[i % nset])
            tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs[i % nset])
            tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs[i % nset], dY=dy)
            free[i % nset].record(main)
            if pipelined and i + ahead < K:
                dedup_ahead(i + ahead)
        torch.cuda.synchronize()
        # one key build per batch: no backward redid its dedup
        assert E.emb_kernel_times(tabs.ctx)["keys"][1] == K
        results.append(P.read_rows(tabs, cfg, u))
        tabs.close()
    assert np.array_equal(results[0][0].view(np.uint32), results[1][0].view(np.uint32))
    assert np.array_equal(results[0][1].view(np.uint32), results[1][1].view(np.uint32))


def test_dedup_ahead_on_second_stream_matches_serial():
    # emb_backward_dedup on a side stream, concurrent with the forward, then
    # the backward (which skips its dedup) and the fused update: bit-identical
    # to the one-stream path
    cfg = W.make_config(2, batch=4096)
    batch = W.make_batch(cfg, k=5)
    dY = W.make_dy(cfg, k=5)
    _say("dedup-ahead cfg2 B=4096")
    ref = P.run_step(cfg, batch, dY, path="fused", sample_untouched=0)
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, dY)
    bufs = tabs.backward_buffers(batch.N, cfg.batch, with_grad=False)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        tabs.dedup(idx, off, cfg.batch, cfg.pool, bufs)
    ev = torch.cuda.Event()
    ev.record(side)
    Y = tabs.forward(idx, off, cfg.batch, cfg.pool)
    main.wait_event(ev)
    tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs)
    tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs, dY=dy)
    torch.cuda.synchronize()
    u, c, inv = P.oracle_dedup(cfg, batch)
    P.check_dedup(bufs, u, c, inv)
    w_new, G_new = P.read_rows(tabs, cfg, ref["keys"])
    assert np.array_equal(w_new.view(np.uint32), ref["w_new"].view(np.uint32))
    assert np.array_equal(G_new.view(np.uint32), ref["G_new"].view(np.uint32))
    # a backward with a different workspace does its own dedup
    bufs2 = tabs.backward_buffers(batch.N, cfg.batch, with_grad=True)
    tabs.dedup(idx, off, cfg.batch, cfg.pool, bufs)
    tabs.backward(idx, off, cfg.batch, cfg.pool, dy, bufs2)
    torch.cuda.synchronize()
    P.check_dedup(bufs2, u, c, inv)
    del Y
    tabs.close()


@pytest.mark.parametrize("cfg_id", [2, 4, 5])
def test_atomic_reduce_matches_oracle(cfg_id):
    # the evidence variant: dedup, then fp32-atomic scatter-add of every
    # lookup's gradient, then the update from the materialised gradient
    cfg = W.make_config(cfg_id, **REDUCED[cfg_id])
    batch = W.make_batch(cfg)
    dY = W.make_dy(cfg)
    _say(f"atomic cfg{cfg_id} N={batch.N}")
    tabs = P.make_tables(cfg)
    idx, off, dy = P.to_dev(batch, dY)
    bufs = tabs.backward_buffers(batch.N, cfg.batch, with_grad=True)
    E.emb_backward_unique_reduce(tabs.ctx, idx, off, cfg.batch, cfg.pool, dy, bufs["ws"], bufs["unique_keys"],
                                 bufs["counts"], bufs["inverse"], bufs["num_unique"], None)
    tabs.atomic_reduce(off, batch.N, cfg.batch, cfg.pool, dy, bufs)
    torch.cuda.synchronize()
    u, c, inv = P.oracle_dedup(cfg, batch)
    U = P.check_dedup(bufs, u, c, inv)
    g_ref, m_ref = P.grad_bounds(cfg, batch, dY, inv, U)
    P.check_grad(bufs["reduced_grad"][:U].cpu().numpy(), g_ref, m_ref)
    w_old = P.stored_init(cfg, u)
    G_old = np.zeros_like(w_old) if cfg.opt == "adagrad" else None
    tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs)
    torch.cuda.synchronize()
    w_new, G_new = P.read_rows(tabs, cfg, u)
    P.check_update(cfg, w_new, G_new, w_old, G_old, g_ref, m_ref)
    tabs.close()
