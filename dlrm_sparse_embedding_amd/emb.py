"""Thin ctypes binding of libemb.so (C ABI declared in include/emb.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory and the current HIP stream. The
functions carry the C names; ``EmbeddingTables`` bundles a context with the
tensors that back it.

``torch`` is imported before the library is loaded so that the library's
``libamdhip64.so.7`` resolves to the HIP runtime torch already holds (one
runtime per process). If ``libemb.so`` has not been built, loading raises --
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libemb.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "emb.h")

EMB_OK = 0
EMB_E_INVAL = -1
EMB_E_DTYPE = -2
EMB_E_WORKSPACE = -3
EMB_E_HIP = -4
EMB_E_BOUNDS = -5
EMB_E_STATE = -6

EMB_F32, EMB_BF16, EMB_F16 = 0, 1, 2
EMB_I32, EMB_I64 = 0, 1
EMB_POOL_SUM, EMB_POOL_MEAN = 0, 1
EMB_OPT_SGD, EMB_OPT_ADAGRAD = 0, 1
EMB_MAX_SLICES = 4

KERNELS = ["init", "forward", "keys", "sort_hist", "sort_scan", "sort_scatter", "rle", "reduce",
           "combine", "apply", "atomic", "pack", "gather", "hash"]

DTYPE_CODE = {"f32": EMB_F32, "bf16": EMB_BF16, "f16": EMB_F16}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
POOL_CODE = {"sum": EMB_POOL_SUM, "mean": EMB_POOL_MEAN}
OPT_CODE = {"sgd": EMB_OPT_SGD, "adagrad": EMB_OPT_ADAGRAD}


class EmbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"emb error {code}: {msg}")
        self.code = code


EMB_SHARD_TABLE = 0
EMB_SHARD_ROW_CYCLIC = 1
EMB_SHARD_ROW_BLOCK = 2
EMB_MAX_SHARDS = 4096
SHARD_KIND = {"table": EMB_SHARD_TABLE, "row_cyclic": EMB_SHARD_ROW_CYCLIC, "row_block": EMB_SHARD_ROW_BLOCK}


class emb_shard_rule(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("shard", ctypes.c_int32)]


class emb_table_desc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("dim", ctypes.c_int32), ("col_slices", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("weights", ctypes.c_void_p * EMB_MAX_SLICES),
                ("state", ctypes.c_void_p * EMB_MAX_SLICES),
                ("master", ctypes.c_void_p * EMB_MAX_SLICES)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libemb.so once (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m dlrm_sparse_embedding_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.emb_create_tables.argtypes = [ctypes.POINTER(emb_table_desc), i32, ctypes.POINTER(vp)]
    L.emb_create_tables.restype = ctypes.c_int
    L.emb_destroy_tables.argtypes = [vp]
    L.emb_destroy_tables.restype = None
    L.emb_row_offsets.argtypes = [vp, ctypes.POINTER(i64)]
    L.emb_row_offsets.restype = ctypes.c_int
    L.emb_init_uniform.argtypes = [vp, ctypes.c_uint64, vp]
    L.emb_init_uniform.restype = ctypes.c_int
    L.emb_forward_pooled.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp]
    L.emb_forward_pooled.restype = ctypes.c_int
    L.emb_backward_workspace_bytes.argtypes = [vp, i64, i32]
    L.emb_backward_workspace_bytes.restype = sz
    L.emb_backward_unique_reduce.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp, sz, vp, vp, vp,
                                             vp, vp, vp]
    L.emb_backward_unique_reduce.restype = ctypes.c_int
    L.emb_backward_dedup.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, sz, vp, vp, vp, vp, vp]
    L.emb_backward_dedup.restype = ctypes.c_int
    L.emb_backward_atomic_reduce.argtypes = [vp, vp, i32, i64, i32, i32, vp, vp, vp, vp, vp]
    L.emb_backward_atomic_reduce.restype = ctypes.c_int
    L.emb_sparse_update.argtypes = [vp, i32, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp]
    L.emb_sparse_update.restype = ctypes.c_int
    L.emb_forward_pooled_unique.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp, sz, vp, vp]
    L.emb_forward_pooled_unique.restype = ctypes.c_int
    L.emb_hash_bytes.argtypes = [vp]
    L.emb_hash_bytes.restype = sz
    L.emb_hash_attach.argtypes = [vp, vp, sz, vp]
    L.emb_hash_attach.restype = ctypes.c_int
    L.emb_hash_workspace_bytes.argtypes = [vp, i64]
    L.emb_hash_workspace_bytes.restype = sz
    L.emb_hash_translate.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, sz, vp, vp]
    L.emb_hash_translate.restype = ctypes.c_int
    L.emb_hash_translate_noalloc.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp]
    L.emb_hash_translate_noalloc.restype = ctypes.c_int
    L.emb_forward_pooled_hashed.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp]
    L.emb_forward_pooled_hashed.restype = ctypes.c_int
    L.emb_hash_rows_used.argtypes = [vp, vp, vp]
    L.emb_hash_rows_used.restype = ctypes.c_int
    L.emb_set_shard_map.argtypes = [vp, ctypes.POINTER(emb_shard_rule), i32]
    L.emb_set_shard_map.restype = ctypes.c_int
    L.emb_pack_by_shard.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    L.emb_pack_by_shard.restype = ctypes.c_int
    L.emb_last_error.argtypes = []
    L.emb_last_error.restype = ctypes.c_char_p
    L.emb_check_device_error.argtypes = [vp, vp]
    L.emb_check_device_error.restype = ctypes.c_int
    L.emb_set_kernel_timing.argtypes = [vp, i32]
    L.emb_set_kernel_timing.restype = ctypes.c_int
    L.emb_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.emb_kernel_times.restype = ctypes.c_int
    L.emb_probe_blocks.argtypes = []
    L.emb_probe_blocks.restype = i32
    L.emb_probe_reads.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp]
    L.emb_probe_reads.restype = ctypes.c_int
    L.emb_probe_update.argtypes = [vp, i64, vp, vp, i64, i32, vp]
    L.emb_probe_update.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != EMB_OK:
        raise EmbError(rc, lib().emb_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _itype(t: torch.Tensor) -> int:
    if t.dtype == torch.int32:
        return EMB_I32
    if t.dtype == torch.int64:
        return EMB_I64
    raise ValueError(f"indices/offsets must be int32 or int64, not {t.dtype}")


# ---- C entry points, same names --------------------------------------------

def emb_create_tables(descs) -> int:
    """descs: sequence of emb_table_desc. Returns the context handle."""
    arr = (emb_table_desc * len(descs))(*descs)
    out = ctypes.c_void_p()
    _check(lib().emb_create_tables(arr, len(descs), ctypes.byref(out)))
    return out.value


def emb_destroy_tables(ctx: int) -> None:
    lib().emb_destroy_tables(ctx)


def emb_row_offsets(ctx: int, T: int) -> list:
    buf = (ctypes.c_int64 * (T + 1))()
    _check(lib().emb_row_offsets(ctx, buf))
    return list(buf)


def emb_init_uniform(ctx: int, seed: int, stream=None) -> None:
    _check(lib().emb_init_uniform(ctx, int(seed), _stream(stream)))


def emb_forward_pooled(ctx: int, indices: torch.Tensor, offsets: torch.Tensor, B: int, pool: str,
                       out: torch.Tensor, stream=None) -> None:
    if offsets.dtype != indices.dtype:
        raise ValueError("indices and offsets must share one integer type")
    if out.dtype != torch.float32:
        raise ValueError("out must be fp32")
    _check(lib().emb_forward_pooled(ctx, _ptr(indices), _ptr(offsets), _itype(indices),
                                    int(indices.numel()), int(B), POOL_CODE[pool], _ptr(out),
                                    _stream(stream)))


def emb_backward_workspace_bytes(ctx: int, N: int, B: int) -> int:
    return int(lib().emb_backward_workspace_bytes(ctx, int(N), int(B)))


def emb_backward_unique_reduce(ctx: int, indices, offsets, B: int, pool: str, dY, ws, unique_keys,
                               counts, inverse, num_unique, reduced_grad=None, stream=None) -> None:
    if offsets.dtype != indices.dtype:
        raise ValueError("indices and offsets must share one integer type")
    _check(lib().emb_backward_unique_reduce(
        ctx, _ptr(indices), _ptr(offsets), _itype(indices), int(indices.numel()), int(B),
        POOL_CODE[pool], _ptr(dY), _ptr(ws), int(ws.numel() * ws.element_size()), _ptr(unique_keys),
        _ptr(counts), _ptr(inverse), _ptr(num_unique), _ptr(reduced_grad), _stream(stream)))


def emb_backward_dedup(ctx: int, indices, offsets, B: int, pool: str, ws, unique_keys, counts, inverse,
                       num_unique, stream=None) -> None:
    if offsets.dtype != indices.dtype:
        raise ValueError("indices and offsets must share one integer type")
    _check(lib().emb_backward_dedup(
        ctx, _ptr(indices), _ptr(offsets), _itype(indices), int(indices.numel()), int(B),
        POOL_CODE[pool], _ptr(ws), int(ws.numel() * ws.element_size()), _ptr(unique_keys),
        _ptr(counts), _ptr(inverse), _ptr(num_unique), _stream(stream)))


def emb_backward_atomic_reduce(ctx: int, offsets, N: int, B: int, pool: str, dY, inverse, num_unique,
                               reduced_grad, stream=None) -> None:
    _check(lib().emb_backward_atomic_reduce(
        ctx, _ptr(offsets), _itype(offsets), int(N), int(B), POOL_CODE[pool], _ptr(dY), _ptr(inverse),
        _ptr(num_unique), _ptr(reduced_grad), _stream(stream)))


def emb_sparse_update(ctx: int, opt: str, lr: float, eps: float, ws, dY=None, reduced_grad=None,
                      stream=None) -> None:
    _check(lib().emb_sparse_update(ctx, OPT_CODE[opt], float(lr), float(eps), _ptr(ws), _ptr(dY),
                                   _ptr(reduced_grad), _stream(stream)))


def emb_check_device_error(ctx: int, stream=None) -> None:
    _check(lib().emb_check_device_error(ctx, _stream(stream)))


def emb_set_kernel_timing(ctx: int, enable: bool) -> None:
    _check(lib().emb_set_kernel_timing(ctx, 1 if enable else 0))


def emb_forward_pooled_unique(ctx: int, indices, offsets, B: int, pool: str, ws, rows_buf, out,
                              stream=None) -> None:
    if offsets.dtype != indices.dtype:
        raise ValueError("indices and offsets must share one integer type")
    _check(lib().emb_forward_pooled_unique(
        ctx, _ptr(indices), _ptr(offsets), _itype(indices), int(indices.numel()), int(B), POOL_CODE[pool],
        _ptr(ws), _ptr(rows_buf), int(rows_buf.numel() * rows_buf.element_size()) if rows_buf is not None else 0,
        _ptr(out), _stream(stream)))


def emb_hash_bytes(ctx: int) -> int:
    return int(lib().emb_hash_bytes(ctx))


def emb_hash_attach(ctx: int, mem, stream=None) -> None:
    _check(lib().emb_hash_attach(ctx, _ptr(mem), int(mem.numel() * mem.element_size()), _stream(stream)))


def emb_hash_workspace_bytes(ctx: int, N: int) -> int:
    return int(lib().emb_hash_workspace_bytes(ctx, int(N)))


def emb_hash_translate(ctx: int, ids, offsets, B: int, insert: bool, ws, rows_out, stream=None) -> None:
    """ids: int64 [N]; rows_out: [N] of the offsets' integer type."""
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    if rows_out.dtype != offsets.dtype:
        raise ValueError("rows_out must have the offsets' integer type")
    _check(lib().emb_hash_translate(ctx, _ptr(ids), _ptr(offsets), _itype(offsets), int(ids.numel()), int(B),
                                    1 if insert else 0, _ptr(ws), int(ws.numel() * ws.element_size()),
                                    _ptr(rows_out), _stream(stream)))


def emb_hash_translate_noalloc(ctx: int, ids, offsets, B: int, insert: bool, rows_out, stream=None) -> None:
    """emb_hash_translate without a workspace (the library's fixed scratch)."""
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    if rows_out.dtype != offsets.dtype:
        raise ValueError("rows_out must have the offsets' integer type")
    _check(lib().emb_hash_translate_noalloc(ctx, _ptr(ids), _ptr(offsets), _itype(offsets), int(ids.numel()),
                                            int(B), 1 if insert else 0, _ptr(rows_out), _stream(stream)))


def emb_forward_pooled_hashed(ctx: int, ids, offsets, B: int, pool: str, out, stream=None) -> None:
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    _check(lib().emb_forward_pooled_hashed(ctx, _ptr(ids), _ptr(offsets), _itype(offsets), int(ids.numel()),
                                           int(B), POOL_CODE[pool], _ptr(out), _stream(stream)))


def emb_hash_rows_used(ctx: int, used, stream=None) -> None:
    _check(lib().emb_hash_rows_used(ctx, _ptr(used), _stream(stream)))


def emb_set_shard_map(ctx: int, rules, num_shards: int) -> None:
    """rules: one (kind, shard) per table, kind an EMB_SHARD_* code or a
    SHARD_KIND name."""
    arr = (emb_shard_rule * len(rules))()
    for t, (kind, shard) in enumerate(rules):
        arr[t].kind = SHARD_KIND.get(kind, kind) if isinstance(kind, str) else int(kind)
        arr[t].shard = int(shard)
    _check(lib().emb_set_shard_map(ctx, arr, int(num_shards)))


def emb_pack_by_shard(ctx: int, ws, dY, send_keys, send_offsets, slot_of_unique, send_grad,
                      stream=None) -> None:
    _check(lib().emb_pack_by_shard(ctx, _ptr(ws), _ptr(dY), _ptr(send_keys), _ptr(send_offsets),
                                   _ptr(slot_of_unique), _ptr(send_grad), _stream(stream)))


def emb_probe_blocks() -> int:
    return int(lib().emb_probe_blocks())


def emb_probe_reads(buf, nrows: int, stride: int, xcd_local: bool, reads: int, sink, stream=None,
                    row_bytes: int = 512) -> None:
    """Measurement aid: random 256- or 512-byte row reads (see include/emb.h)."""
    _check(lib().emb_probe_reads(_ptr(buf), int(nrows), int(stride), 1 if xcd_local else 0, int(reads),
                                 int(row_bytes), _ptr(sink), _stream(stream)))


def emb_probe_update(src, nsrc: int, a, b, nrows: int, items: int, stream=None) -> None:
    """Measurement aid: the fused update's random row read/write mix (see include/emb.h)."""
    _check(lib().emb_probe_update(_ptr(src), int(nsrc), _ptr(a), _ptr(b), int(nrows), int(items), _stream(stream)))


def emb_probe_update_bytes(items: int) -> int:
    """Bytes one emb_probe_update launch moves (include/emb.h)."""
    n3 = 34 * (items // 50) + min(items % 50, 34)
    return 512 * (3 * n3 + 2 * (items - n3) + 4 * items)


def emb_kernel_times(ctx: int) -> dict:
    ms = (ctypes.c_double * len(KERNELS))()
    n = (ctypes.c_int64 * len(KERNELS))()
    _check(lib().emb_kernel_times(ctx, ms, n))
    return {k: (ms[i], int(n[i])) for i, k in enumerate(KERNELS)}


# ---- convenience: a context with the tensors behind it ---------------------

@dataclass
class TableSpec:
    rows: int
    dim: int
    dtype: str = "f32"
    col_slices: int = 1


class EmbeddingTables:
    """Allocates this GPU's tables (and Adagrad state, and fp32 master weights
    for low-precision tables if asked) as torch tensors, registers them with
    emb_create_tables and forwards the calls."""

    def __init__(self, specs, with_state: bool, device="cuda", with_master: bool = False):
        specs = list(specs)
        self.specs = specs
        self.T = len(specs)
        self.dim = specs[0].dim
        self.dtype = specs[0].dtype
        self.col_slices = specs[0].col_slices
        self.weights = []   # [t][s] tensors [rows, dim/col_slices]
        self.state = []     # [t][s] fp32 tensors or None
        self.master = []    # [t][s] fp32 tensors or None
        descs = []
        for sp in specs:
            dsl = sp.dim // sp.col_slices
            ws = [torch.empty((sp.rows, dsl), dtype=TORCH_DTYPE[sp.dtype], device=device)
                  for _ in range(sp.col_slices)]
            ss = ([torch.empty((sp.rows, dsl), dtype=torch.float32, device=device)
                   for _ in range(sp.col_slices)] if with_state else None)
            ms = ([torch.empty((sp.rows, dsl), dtype=torch.float32, device=device)
                   for _ in range(sp.col_slices)] if with_master else None)
            self.weights.append(ws)
            self.state.append(ss)
            self.master.append(ms)
            d = emb_table_desc()
            d.rows, d.dim, d.col_slices, d.dtype, d.reserved = sp.rows, sp.dim, sp.col_slices, DTYPE_CODE[sp.dtype], 0
            for s in range(sp.col_slices):
                d.weights[s] = ws[s].data_ptr()
                d.state[s] = ss[s].data_ptr() if ss else None
                d.master[s] = ms[s].data_ptr() if ms else None
            descs.append(d)
        self.ctx = emb_create_tables(descs)
        self.row_offset = emb_row_offsets(self.ctx, self.T)

    def close(self) -> None:
        if self.ctx:
            emb_destroy_tables(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def init_uniform(self, seed: int, stream=None) -> None:
        emb_init_uniform(self.ctx, seed, stream)

    def forward(self, indices, offsets, B: int, pool: str, out=None, stream=None):
        if out is None:
            out = torch.empty((B, self.T * self.dim), dtype=torch.float32, device=indices.device)
        emb_forward_pooled(self.ctx, indices, offsets, B, pool, out, stream)
        return out

    def workspace(self, N: int, B: int, device="cuda"):
        nbytes = emb_backward_workspace_bytes(self.ctx, N, B)
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)

    def backward_buffers(self, N: int, B: int, with_grad: bool, device="cuda"):
        """Device outputs of emb_backward_unique_reduce sized by N."""
        cap = max(N, 1)
        return dict(
            ws=self.workspace(N, B, device),
            unique_keys=torch.empty(cap, dtype=torch.int32, device=device),  # uint32 bits
            counts=torch.empty(cap, dtype=torch.int32, device=device),
            inverse=torch.empty(cap, dtype=torch.int32, device=device),
            num_unique=torch.empty(1, dtype=torch.int32, device=device),
            reduced_grad=(torch.empty((cap, self.dim), dtype=torch.float32, device=device)
                          if with_grad else None),
        )

    def backward(self, indices, offsets, B: int, pool: str, dY, bufs, stream=None) -> None:
        emb_backward_unique_reduce(self.ctx, indices, offsets, B, pool, dY, bufs["ws"],
                                   bufs["unique_keys"], bufs["counts"], bufs["inverse"],
                                   bufs["num_unique"], bufs["reduced_grad"], stream)

    def dedup(self, indices, offsets, B: int, pool: str, bufs, stream=None) -> None:
        emb_backward_dedup(self.ctx, indices, offsets, B, pool, bufs["ws"], bufs["unique_keys"],
                           bufs["counts"], bufs["inverse"], bufs["num_unique"], stream)

    def atomic_reduce(self, offsets, N: int, B: int, pool: str, dY, bufs, stream=None) -> None:
        emb_backward_atomic_reduce(self.ctx, offsets, N, B, pool, dY, bufs["inverse"], bufs["num_unique"],
                                   bufs["reduced_grad"], stream)

    def update(self, opt: str, lr: float, eps: float, bufs, dY=None, stream=None) -> None:
        emb_sparse_update(self.ctx, opt, lr, eps, bufs["ws"], dY, bufs["reduced_grad"], stream)

    def check_device_error(self, stream=None) -> None:
        emb_check_device_error(self.ctx, stream)

    def logical_rows(self, t: int, rows) -> torch.Tensor:
        """Rows of table t gathered from its column slices, [len(rows), dim]
        in the storage dtype (a read-back helper for checks)."""
        r = torch.as_tensor(rows, dtype=torch.int64, device=self.weights[t][0].device)
        return torch.cat([w.index_select(0, r) for w in self.weights[t]], dim=1)

    def logical_state(self, t: int, rows) -> torch.Tensor:
        r = torch.as_tensor(rows, dtype=torch.int64, device=self.weights[t][0].device)
        return torch.cat([s.index_select(0, r) for s in self.state[t]], dim=1)

    def unique_rows_buffer(self, N: int, device="cuda") -> torch.Tensor:
        """Capacity for emb_forward_pooled_unique: N rows of the storage type."""
        return torch.empty((max(N, 1), self.dim), dtype=TORCH_DTYPE[self.dtype], device=device)

    def forward_unique(self, indices, offsets, B: int, pool: str, bufs, rows_buf, out=None, stream=None):
        """Unique-first forward; needs self.dedup(...) of the same lookups first."""
        if out is None:
            out = torch.empty((B, self.T * self.dim), dtype=torch.float32, device=indices.device)
        emb_forward_pooled_unique(self.ctx, indices, offsets, B, pool, bufs["ws"], rows_buf, out, stream)
        return out

    def hash_attach(self, device="cuda", stream=None) -> None:
        """Allocates the id -> row maps of every table and empties them."""
        self.hash_mem = torch.empty(emb_hash_bytes(self.ctx), dtype=torch.uint8, device=device)
        emb_hash_attach(self.ctx, self.hash_mem, stream)

    def hash_translate(self, ids, offsets, B: int, insert: bool, stream=None):
        rows = torch.empty(max(ids.numel(), 1), dtype=offsets.dtype, device=ids.device)[:ids.numel()]
        ws = torch.empty(max(emb_hash_workspace_bytes(self.ctx, ids.numel()), 256), dtype=torch.uint8,
                         device=ids.device)
        emb_hash_translate(self.ctx, ids, offsets, B, insert, ws, rows, stream)
        if stream is not None:
            # the allocator must not hand ws (or rows) to another tensor while
            # the translation still runs on a stream other than the current one
            st = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
            if st != torch.cuda.current_stream(ids.device):
                ws.record_stream(st)
                rows.record_stream(st)
        return rows

    def forward_hashed(self, ids, offsets, B: int, pool: str, out=None, stream=None):
        if out is None:
            out = torch.empty((B, self.T * self.dim), dtype=torch.float32, device=ids.device)
        emb_forward_pooled_hashed(self.ctx, ids, offsets, B, pool, out, stream)
        return out

    def hash_rows_used(self, stream=None):
        used = torch.empty(self.T, dtype=torch.int32, device=self.weights[0][0].device)
        emb_hash_rows_used(self.ctx, used, stream)
        return used

    def set_shard_map(self, rules, num_shards: int) -> None:
        emb_set_shard_map(self.ctx, rules, num_shards)

    def pack_buffers(self, N: int, num_shards: int, with_grad: bool, device="cuda"):
        cap = max(N, 1)
        return dict(
            send_keys=torch.empty(cap, dtype=torch.int32, device=device),   # uint32 bits
            send_offsets=torch.empty(num_shards + 1, dtype=torch.int32, device=device),
            slot_of_unique=torch.empty(cap, dtype=torch.int32, device=device),
            send_grad=(torch.empty((cap, self.dim), dtype=torch.float32, device=device)
                       if with_grad else None),
        )

    def pack(self, bufs, pbufs, dY=None, stream=None) -> None:
        emb_pack_by_shard(self.ctx, bufs["ws"], dY, pbufs["send_keys"], pbufs["send_offsets"],
                          pbufs["slot_of_unique"], pbufs["send_grad"] if dY is not None else None, stream)

    def logical_master(self, t: int, rows) -> torch.Tensor:
        r = torch.as_tensor(rows, dtype=torch.int64, device=self.weights[t][0].device)
        return torch.cat([m.index_select(0, r) for m in self.master[t]], dim=1)
