"""C-ABI checks that need no GPU: the library loads (into the process's one
HIP runtime, torch's), exports every entry point include/emb.h declares, and
rejects invalid calls with the documented status codes before touching the
device."""
import ctypes
import re

import pytest
import torch  # noqa: F401  (the binding loads torch's HIP runtime first)

from dlrm_sparse_embedding_amd import emb as E

FAKE = 0x100000  # 16-byte aligned non-null "device" pointer; never dereferenced here


def _declared_functions():
    src = open(E.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(emb_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 12
    L = E.lib()
    for n in names:
        assert hasattr(L, n), n


def test_header_constants_match_binding():
    src = open(E.HEADER_PATH).read()
    consts = dict((k, int(v.strip("()"))) for k, v in re.findall(r"#define\s+(EMB_[A-Z0-9_]+)\s+(\(?-?\d+\)?)", src))
    for k, v in consts.items():
        if hasattr(E, k):
            assert getattr(E, k) == v, k
    kids = [k for k in consts if k.startswith("EMB_K_") and k != "EMB_K_COUNT"]
    assert consts["EMB_K_COUNT"] == len(E.KERNELS) == len(kids)


def _desc(rows=100, dim=16, slices=1, dtype=E.EMB_F32, state=True, master=False):
    d = E.emb_table_desc()
    d.rows, d.dim, d.col_slices, d.dtype, d.reserved = rows, dim, slices, dtype, 0
    for s in range(min(slices, E.EMB_MAX_SLICES)):
        d.weights[s] = FAKE + 0x1000 * s
        d.state[s] = (FAKE + 0x100000 + 0x1000 * s) if state else None
        d.master[s] = (FAKE + 0x200000 + 0x1000 * s) if master else None
    return d


def _with(d, field, s, value):
    getattr(d, field)[s] = value
    return d


def _create(descs):
    arr = (E.emb_table_desc * len(descs))(*descs)
    out = ctypes.c_void_p()
    rc = E.lib().emb_create_tables(arr, len(descs), ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("descs,code", [
    ([], E.EMB_E_INVAL),
    ([_desc(dtype=7)], E.EMB_E_DTYPE),
    ([_desc(dim=96, slices=5)], E.EMB_E_INVAL),            # slices > EMB_MAX_SLICES
    ([_desc(dim=100, slices=3)], E.EMB_E_INVAL),           # dim % slices
    ([_desc(dim=6)], E.EMB_E_INVAL),                       # 24-byte rows
    ([_desc(dim=16), _desc(dim=32)], E.EMB_E_INVAL),       # mixed dims
    ([_desc(rows=0)], E.EMB_E_INVAL),
    ([_desc(rows=1 << 31), _desc(rows=1 << 31)], E.EMB_E_INVAL),  # sum of rows >= 2^32 - 1
    ([_desc(state=True), _desc(state=False)], E.EMB_E_INVAL),
    ([_desc(dim=512)], E.EMB_E_INVAL),                     # > 1024-byte rows
    ([_desc(master=True)], E.EMB_E_INVAL),                 # fp32 master on an fp32 table
    ([_desc(dtype=E.EMB_BF16, master=True), _desc(dtype=E.EMB_BF16)], E.EMB_E_INVAL),  # master: all or none
    ([_with(_desc(dim=32, slices=2, dtype=E.EMB_F16, master=True), "master", 1, None)], E.EMB_E_INVAL),
    ([_with(_desc(dtype=E.EMB_BF16, master=True), "master", 0, FAKE + 0x200008)], E.EMB_E_INVAL),  # unaligned
    ([_with(_desc(), "weights", 1, FAKE + 0x4000)], E.EMB_E_INVAL),  # pointer beyond col_slices
])
def test_create_rejects(descs, code):
    rc, ctx = _create(descs)
    assert rc == code
    assert ctx is None
    assert E.lib().emb_last_error().decode() != ""


def test_create_accepts_16_byte_slice_rows():
    for d in (_desc(dim=8, dtype=E.EMB_BF16), _desc(dim=4), _desc(dim=128, slices=4, dtype=E.EMB_F16),
              _desc(dim=128, slices=4, dtype=E.EMB_F16, master=True), _desc(dtype=E.EMB_BF16, master=True)):
        rc, ctx = _create([d])
        assert rc == E.EMB_OK
        E.emb_destroy_tables(ctx)


def test_create_null_weights():
    d = _desc()
    d.weights[0] = None
    assert _create([d])[0] == E.EMB_E_INVAL


def test_probe_rejects_bad_arguments_before_any_launch():
    # the read-ceiling probe validates on the host and launches nothing on error
    L = E.lib()
    assert E.emb_probe_blocks() == 2048
    good = dict(nrows=4096, stride=512, local=1, reads=60, row_bytes=512)
    def call(buf=FAKE, sink=FAKE, **kw):
        a = {**good, **kw}
        return L.emb_probe_reads(buf, a["nrows"], a["stride"], a["local"], a["reads"], a["row_bytes"], sink, None)
    assert call(buf=None) == E.EMB_E_INVAL
    assert call(sink=None) == E.EMB_E_INVAL
    assert call(buf=FAKE + 4) == E.EMB_E_INVAL       # misaligned
    assert call(nrows=7) == E.EMB_E_INVAL
    assert call(nrows=1 << 32) == E.EMB_E_INVAL
    assert call(stride=256) == E.EMB_E_INVAL
    assert call(stride=520) == E.EMB_E_INVAL         # not a multiple of 16
    assert call(reads=6) == E.EMB_E_INVAL
    assert call(reads=0) == E.EMB_E_INVAL
    assert call(reads=65540) == E.EMB_E_INVAL
    assert call(row_bytes=128) == E.EMB_E_INVAL
    assert call(row_bytes=256, stride=128) == E.EMB_E_INVAL   # stride shorter than a row


def test_update_probe_rejects_bad_arguments_before_any_launch():
    L = E.lib()
    good = dict(nsrc=1000, nrows=5000, items=100)
    def call(src=FAKE, a=FAKE, b=FAKE, **kw):
        k = {**good, **kw}
        return L.emb_probe_update(src, k["nsrc"], a, b, k["nrows"], k["items"], None)
    assert call(src=None) == E.EMB_E_INVAL
    assert call(a=None) == E.EMB_E_INVAL
    assert call(b=None) == E.EMB_E_INVAL
    assert call(b=FAKE + 8) == E.EMB_E_INVAL        # misaligned
    assert call(nsrc=0) == E.EMB_E_INVAL
    assert call(nrows=1 << 32) == E.EMB_E_INVAL
    assert call(items=0) == E.EMB_E_INVAL
    assert E.emb_probe_update_bytes(100) == 512 * (3 * 68 + 2 * 32 + 400)


def test_valid_context_host_only_calls():
    rc, ctx = _create([_desc(rows=1000), _desc(rows=5000)])
    assert rc == E.EMB_OK and ctx
    assert E.lib().emb_last_error().decode() == ""
    assert E.emb_row_offsets(ctx, 2) == [0, 1000, 6000]
    w1 = E.emb_backward_workspace_bytes(ctx, 100, 10)
    w2 = E.emb_backward_workspace_bytes(ctx, 100000, 10)
    assert 0 < w1 < w2 and w1 % 256 == 0
    assert E.emb_backward_workspace_bytes(ctx, -1, 10) == 0
    # timing bookkeeping with nothing recorded
    E.emb_set_kernel_timing(ctx, True)
    t = E.emb_kernel_times(ctx)
    assert all(v == (0.0, 0) for v in t.values())
    L = E.lib()
    vp = ctypes.c_void_p
    # forward: bad enums and sizes, rejected before any device call
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 3, 10, 5, 0, FAKE, None) == E.EMB_E_DTYPE
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 0, 10, 5, 9, FAKE, None) == E.EMB_E_DTYPE
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 0, 1 << 31, 5, 0, FAKE, None) == E.EMB_E_INVAL
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 0, -1, 5, 0, FAKE, None) == E.EMB_E_INVAL
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 0, 10, 0, 0, FAKE, None) == E.EMB_E_INVAL
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 0, 0, 0, 0, FAKE, None) == E.EMB_OK   # nothing to do
    assert L.emb_forward_pooled(ctx, FAKE, FAKE, 0, 10, 5, 0, FAKE + 4, None) == E.EMB_E_INVAL  # misaligned out
    # backward: workspace too small
    need = E.emb_backward_workspace_bytes(ctx, 10, 5)
    rc = L.emb_backward_unique_reduce(ctx, FAKE, FAKE, 0, 10, 5, 0, FAKE, FAKE, need - 1, FAKE, FAKE, FAKE,
                                      FAKE, None, None)
    assert rc == E.EMB_E_WORKSPACE
    rc = L.emb_backward_unique_reduce(ctx, FAKE, FAKE, 0, 10, 5, 0, FAKE, FAKE + 16, need, FAKE, FAKE, FAKE,
                                      FAKE, None, None)
    assert rc == E.EMB_E_INVAL   # misaligned ws
    # update: no backward yet -> call order error; bad optimizer
    assert L.emb_sparse_update(ctx, 0, 0.01, 0.0, FAKE, FAKE, None, None) == E.EMB_E_STATE
    assert L.emb_sparse_update(ctx, 5, 0.01, 0.0, FAKE, FAKE, None, None) == E.EMB_E_DTYPE
    E.emb_destroy_tables(ctx)


def test_adagrad_without_state_rejected():
    rc, ctx = _create([_desc(state=False)])
    assert rc == E.EMB_OK
    assert E.lib().emb_sparse_update(ctx, E.EMB_OPT_ADAGRAD, 0.01, 1e-8, FAKE, FAKE, None, None) == E.EMB_E_INVAL
    E.emb_destroy_tables(ctx)


def test_binding_raises_with_message():
    with pytest.raises(E.EmbError) as ei:
        E.emb_create_tables([_desc(dtype=9)])
    assert ei.value.code == E.EMB_E_DTYPE and "dtype" in str(ei.value)


def test_shard_map_validation():
    rc, ctx = _create([_desc(rows=1000), _desc(rows=5000)])
    assert rc == E.EMB_OK
    L = E.lib()
    def setmap(rules, S):
        arr = (E.emb_shard_rule * len(rules))()
        for t, (k, s) in enumerate(rules):
            arr[t].kind, arr[t].shard = k, s
        return L.emb_set_shard_map(ctx, arr, S)
    assert setmap([(E.EMB_SHARD_TABLE, 0), (E.EMB_SHARD_ROW_CYCLIC, 3)], 4) == E.EMB_OK
    assert setmap([(E.EMB_SHARD_ROW_BLOCK, 0), (E.EMB_SHARD_ROW_BLOCK, 0)], E.EMB_MAX_SHARDS) == E.EMB_OK
    assert setmap([(E.EMB_SHARD_TABLE, 4), (E.EMB_SHARD_TABLE, 0)], 4) == E.EMB_E_INVAL      # shard >= S
    assert setmap([(E.EMB_SHARD_ROW_CYCLIC, -1), (E.EMB_SHARD_TABLE, 0)], 4) == E.EMB_E_INVAL
    assert setmap([(E.EMB_SHARD_ROW_BLOCK, 1), (E.EMB_SHARD_TABLE, 0)], 4) == E.EMB_E_INVAL  # block takes 0
    assert setmap([(7, 0), (E.EMB_SHARD_TABLE, 0)], 4) == E.EMB_E_INVAL                      # unknown kind
    assert setmap([(E.EMB_SHARD_TABLE, 0)] * 2, 0) == E.EMB_E_INVAL
    assert setmap([(E.EMB_SHARD_TABLE, 0)] * 2, E.EMB_MAX_SHARDS + 1) == E.EMB_E_INVAL
    # packing needs a backward on this context first (no device work is started)
    rc = L.emb_pack_by_shard(ctx, FAKE, None, FAKE, FAKE, FAKE, None, None)
    assert rc == E.EMB_E_STATE
    E.emb_destroy_tables(ctx)


def test_pack_needs_shard_map():
    rc, ctx = _create([_desc(rows=10)])
    assert E.lib().emb_pack_by_shard(ctx, FAKE, None, FAKE, FAKE, FAKE, None, None) == E.EMB_E_STATE
    assert "shard map" in E.lib().emb_last_error().decode()
    E.emb_destroy_tables(ctx)


def test_unique_forward_needs_dedup_ahead():
    rc, ctx = _create([_desc(rows=10)])
    rc = E.lib().emb_forward_pooled_unique(ctx, FAKE, FAKE, E.EMB_I32, 4, 4, 0, FAKE, FAKE, 1 << 20, FAKE, None)
    assert rc == E.EMB_E_STATE
    E.emb_destroy_tables(ctx)
