"""Plain, slow, obviously-correct CPU oracle of the pooled-embedding path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product library. It
shares no code, header, table or constant with the HIP path; the only thing
both sides consume in common is the seeded input generator
(``dlrm_sparse_embedding_amd.workloads``), which holds none of this arithmetic.

What is computed, and where the sources define it
-----------------------------------------------
* Pooled forward -- "Merlin HugeCTR: GPU-accelerated recommender system
  training and inference" (GTC 2022 deck), slide "COMMON EMBEDDING PRIMITIVES":
  (1) table lookup, (2) pooling/reduction of a multi-hot feature, (3)
  concatenation of the pooled vectors; NVIDIA Merlin blog, HugeCTR section:
  the features of one slot are each mapped to a vector, then reduced to one
  vector. Written out as: for every bag (table t, sample b), the sum (or mean)
  of the stored rows W_t[idx] over the bag's CSR range, placed at
  Y[b, t*D:(t+1)*D]. Accumulated in float64, rounded once to fp32.
* Key dedup -- EMBark (RecSys'24 article, section on embedding clusters):
  reduction-based and unique-based compression. Read here, applied to one
  GPU's share, as: form the global key g = row_offset[t] + idx for every
  lookup, and take the sorted distinct keys, their multiplicities and each
  lookup's index into them (``np.unique``).
* Gradient -- the plain definition: the dense scatter-add of every lookup's
  upstream gradient (times 1/L for mean pooling) into its row, in float64,
  rounded once to fp32. Unique-then-reduce reaches the same value up to fp32
  summation order.
* Optimizer -- GTC 2022 deck, slide "WEIGHT CONVERSION FOR MIXED PRECISION
  TRAINING": the optimizer computes in FP32. SGD: w - lr*g. Adagrad
  (element-wise, accumulator starts at 0): G' = G + g*g,
  w' = w - (lr*g) / (sqrt(G') + eps). Every operation is a separately rounded
  fp32 operation, in exactly that order. The result is rounded to the storage
  type with round-to-nearest-even (bf16/fp16); the stored low-precision value
  is the only copy of the weight.
* FP32 master weights (same slide): read as the scheme in which the optimizer
  keeps an fp32 master copy of every low-precision table and, each iteration,
  updates the master in fp32 and casts it to the low-precision weights the
  lookups read. Written out as: m' = the fp32 optimizer step of m, and the
  stored copy = round-to-nearest-even(m'). The stored copy is never read by
  the update.
* Routing to shards -- EMBark (RecSys'24 article): tables are split into
  shards (its 3D sharding tuple; model parallelism in the GTC 2022 deck,
  slide "CHALLENGES OF EMBEDDING LAYER"), and reduction-based / unique-based
  clusters send each distinct key, and its reduced gradient, once. Read here,
  for one GPU's share, as the step before the exchange: each unique key gets
  the shard that owns its (table, row) under a per-table rule (whole table on
  one shard; rows dealt cyclically; rows in S contiguous blocks), and the
  unique keys (with their reduced gradients) are grouped by destination
  shard, keys ascending inside a group.
* Hash-keyed lookup -- GTC 2022 deck, slide "HUGECTR EMBEDDING LAYER" (a GPU
  hash table lookup fused with the reduction and concatenation), and the
  dynamic embedding of the Sparse Operation Kit 2.0 article: feature ids are
  arbitrary 64-bit values, and each table maps them to its rows. Read here
  as: an id a table has not seen gets, when insertion is on, the table's
  next free row, ids taken in order of first appearance in the CSR; once a
  table's rows are used up, new ids get no row (their lookups pool to
  nothing; rows are never freed, so such an id never gets one); with
  insertion off, unseen ids get no row.
* A lookup that finds no row (a hashed id without one, or an index outside
  its table) -- the pages do not say how it pools. Read here as: it adds
  nothing, and it is still one of its bag's lookups, so mean pooling divides
  by the bag length the offsets give (forward), and every lookup of the bag
  scales its gradient by 1/that length (backward); the row-less lookup itself
  has no gradient row.
* Untouched rows -- a dense step with g = 0 and G = 0 leaves w and G bit for
  bit unchanged, so only touched rows are computed.
* Table contents -- synthetic: each element is a counter hash of (seed, table,
  row*D + col) through SplitMix64 (Steele, Lea & Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014), mapped to U(-0.05, 0.05) by
  one fp32 multiply, then rounded to the storage type.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "splitmix64", "init_values", "bf16_bits_rne", "bf16_bits_to_f32", "f16_rne",
    "to_storage", "TouchedRows", "pooled_forward", "global_keys", "dedup",
    "bag_of_positions", "reduced_grad", "sgd_step", "adagrad_step",
    "update_rows", "update_rows_master", "SHARD_TABLE", "SHARD_ROW_CYCLIC", "SHARD_ROW_BLOCK",
    "shard_of_keys", "pack_by_shard", "HashTables", "pooled_forward_hashed",
]

_U64 = np.uint64
_MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# Synthetic table contents
# ---------------------------------------------------------------------------

def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output for counter value(s) ``x`` (uint64): add the golden
    gamma 0x9E3779B97F4A7C15, then the variant-13 mix (xor-shift 30, multiply
    0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB, xor-shift
    31). Arithmetic wraps modulo 2^64."""
    z = np.asarray(x, dtype=_U64)
    with np.errstate(over="ignore"):
        z = z + _U64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> _U64(30))) * _U64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> _U64(27))) * _U64(0x94D049BB133111EB)
        z = z ^ (z >> _U64(31))
    return z


_INIT_SCALE = np.float32(np.float32(0.1) * np.float32(2.0 ** -24))


def init_values(seed: int, t: int, rows: np.ndarray, D: int, cols: np.ndarray | None = None) -> np.ndarray:
    """fp32 initial value of elements (t, row, col), before storage rounding.

    counter = seed XOR (t << 40) XOR (row*D + col); h = splitmix64(counter);
    v = (h >> 40) - 2^23 (an integer in [-2^23, 2^23), exact in fp32);
    w = fp32(v) * fp32(0.1 * 2^-24)  -- one rounded multiply, |w| <= 0.05.
    Returns [len(rows), D] (or [len(rows), len(cols)])."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 1)
    cc = np.arange(D, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64)
    lin = (rows * D + cc.reshape(1, -1)).astype(_U64)
    ctr = _U64(seed) ^ (_U64(t) << _U64(40)) ^ lin
    h = splitmix64(ctr)
    v = (h >> _U64(40)).astype(np.int64) - (1 << 23)
    return v.astype(np.float32) * _INIT_SCALE


# ---------------------------------------------------------------------------
# Storage rounding (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern of fp32 ``x`` rounded to nearest-even. NaN stays
    NaN (quiet); overflow rounds to +-inf as RNE dictates."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(nan, (b >> np.uint64(16)) | np.uint64(0x0040), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def f16_rne(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 of fp32 ``x``, round to nearest-even (numpy's cast)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value actually stored for fp32 ``x`` in storage type ``dtype``,
    returned widened to fp32 (exactly representable)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "bf16":
        return bf16_bits_to_f32(bf16_bits_rne(x))
    if dtype == "f16":
        return f16_rne(x).astype(np.float32)
    raise ValueError(dtype)


class TouchedRows:
    """Stored contents of table t restricted to the rows a batch touches, so
    that a 53 GB table never has to exist on the host. Indexing with row ids
    returns their stored values (fp32) -- the same values a full table holds."""

    def __init__(self, seed: int, t: int, D: int, dtype: str, rows: np.ndarray):
        self.rows = np.unique(np.asarray(rows, dtype=np.int64))
        self.values = to_storage(init_values(seed, t, self.rows, D), dtype)
        self.D = D

    def __getitem__(self, r):
        r = np.asarray(r, dtype=np.int64)
        pos = np.searchsorted(self.rows, r)
        if r.size and (np.any(pos >= self.rows.size) or np.any(self.rows[np.minimum(pos, self.rows.size - 1)] != r)):
            raise KeyError("row not in the touched set")
        return self.values[pos]


# ---------------------------------------------------------------------------
# Forward: lookup, pooling, concatenation
# ---------------------------------------------------------------------------

def bag_of_positions(offsets: np.ndarray, T: int, B: int) -> np.ndarray:
    """Flat bag id t*B + b of every CSR position (table-major bags)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    lengths = np.diff(offsets)
    return np.repeat(np.arange(T * B, dtype=np.int64), lengths)


def pooled_forward(tables, indices, offsets, T: int, B: int, D: int, pool: str,
                   num_rows=None) -> np.ndarray:
    """Y[b, t*D:(t+1)*D] = sum (or mean) over bag (t, b) of W_t[idx].

    ``tables[t][rows]`` must return the stored rows (any float type). Sums are
    taken in float64 and rounded once to fp32; a mean divides the float64 sum
    by the bag length before that rounding; an empty bag gives zeros.

    ``num_rows`` (rows per table, optional): a lookup whose index lies outside
    [0, num_rows[t]) finds no row -- an index out of range, or a hashed id
    that holds no row (row -1). It adds nothing to its bag's sum, and it still
    counts as one of the bag's lookups: a mean divides by the bag length the
    offsets give, whatever the lookups found. Without ``num_rows`` every index
    must be a row of its table."""
    indices = np.asarray(indices, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    blocks = []
    for t in range(T):
        p0, p1 = int(offsets[t * B]), int(offsets[(t + 1) * B])
        lengths = np.diff(offsets[t * B:(t + 1) * B + 1])
        local_bag = np.repeat(np.arange(B, dtype=np.int64), lengths)
        s = np.zeros((B, D), dtype=np.float64)
        idx = indices[p0:p1]
        if num_rows is not None:
            found = (idx >= 0) & (idx < int(num_rows[t]))
            idx, local_bag = idx[found], local_bag[found]
        if idx.size:
            rows = np.asarray(tables[t][idx], dtype=np.float64).reshape(idx.size, D)
            np.add.at(s, local_bag, rows)
        if pool == "mean":
            nz = lengths > 0
            s[nz] /= lengths[nz].astype(np.float64)[:, None]
        elif pool != "sum":
            raise ValueError(pool)
        blocks.append(s)
    if not blocks:
        return np.zeros((B, 0), dtype=np.float32)
    return np.concatenate(blocks, axis=1).astype(np.float32)


# ---------------------------------------------------------------------------
# Backward: global keys, dedup, reduced gradient
# ---------------------------------------------------------------------------

def global_keys(indices, offsets, row_offset, T: int, B: int) -> np.ndarray:
    """g_i = row_offset[t(i)] + idx_i for every CSR position i (int64)."""
    indices = np.asarray(indices, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    row_offset = np.asarray(row_offset, dtype=np.int64)
    t_of_pos = bag_of_positions(offsets, T, B) // B if B else np.zeros(0, np.int64)
    return row_offset[t_of_pos] + indices


def dedup(g: np.ndarray):
    """(unique_keys ascending, counts, inverse) of the global keys."""
    u, inv, cnt = np.unique(np.asarray(g, dtype=np.int64), return_inverse=True, return_counts=True)
    return u, cnt.astype(np.int64), inv.reshape(-1).astype(np.int64)


def reduced_grad(dY, offsets, T: int, B: int, D: int, pool: str, inverse, U: int,
                 select: np.ndarray | None = None) -> np.ndarray:
    """gU[u] = sum over lookups i with inverse[i] == u of scale_i * dY[b(i), t(i)*D:(t(i)+1)*D],
    scale_i = 1 (sum) or 1/L(bag) (mean). float64 scatter-add, one fp32 rounding.
    A lookup with inverse[i] < 0 found no row: it has no gradient row, and L
    still counts it (the bag length the offsets give, as in the forward).

    ``select`` (sorted unique ids) restricts the result to those rows, in that
    order, for workloads too large to reduce whole."""
    dY = np.asarray(dY, dtype=np.float32)
    offsets = np.asarray(offsets, dtype=np.int64)
    inverse = np.asarray(inverse, dtype=np.int64)
    lengths = np.diff(offsets)
    if select is None:
        out = np.zeros((U, D), dtype=np.float64)
        target_of = None
    else:
        select = np.asarray(select, dtype=np.int64)
        out = np.zeros((select.size, D), dtype=np.float64)
        target_of = select
    for t in range(T):
        p0, p1 = int(offsets[t * B]), int(offsets[(t + 1) * B])
        if p1 == p0:
            continue
        lb = np.repeat(np.arange(B, dtype=np.int64), lengths[t * B:(t + 1) * B])
        inv = inverse[p0:p1]
        has_row = inv >= 0
        lb, inv = lb[has_row], inv[has_row]
        if target_of is not None:
            pos = np.searchsorted(target_of, inv)
            keep = (pos < target_of.size) & (target_of[np.minimum(pos, target_of.size - 1)] == inv)
            lb, dst = lb[keep], pos[keep]
        else:
            dst = inv
        if dst.size == 0:
            continue
        contrib = dY[lb, t * D:(t + 1) * D].astype(np.float64)
        if pool == "mean":
            contrib /= lengths[t * B + lb].astype(np.float64)[:, None]
        np.add.at(out, dst, contrib)
    return out.astype(np.float32)


# ---------------------------------------------------------------------------
# Optimizer (fp32, each operation separately rounded, in this order)
# ---------------------------------------------------------------------------

def sgd_step(w: np.ndarray, g: np.ndarray, lr: float) -> np.ndarray:
    """w' = w - (lr * g)."""
    w = np.asarray(w, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    step = np.float32(lr) * g
    return (w - step).astype(np.float32)


def adagrad_step(w: np.ndarray, G: np.ndarray, g: np.ndarray, lr: float, eps: float):
    """G' = G + g*g;  w' = w - (lr*g) / (sqrt(G') + eps)."""
    w = np.asarray(w, dtype=np.float32)
    G = np.asarray(G, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    gg = g * g
    G1 = (G + gg).astype(np.float32)
    den = (np.sqrt(G1) + np.float32(eps)).astype(np.float32)
    num = np.float32(lr) * g
    w1 = (w - (num / den).astype(np.float32)).astype(np.float32)
    return w1, G1


def update_rows(w_stored: np.ndarray, G: np.ndarray | None, g: np.ndarray, opt: str,
                lr: float, eps: float, dtype: str):
    """One optimizer step on touched rows: widen the stored value, update in
    fp32, round back to the storage type (RNE). Returns (w_stored', G')."""
    w32 = np.asarray(w_stored, dtype=np.float32)
    if opt == "sgd":
        w1, G1 = sgd_step(w32, g, lr), G
    elif opt == "adagrad":
        if G is None:
            raise ValueError("adagrad needs its accumulator")
        w1, G1 = adagrad_step(w32, G, g, lr, eps)
    else:
        raise ValueError(opt)
    return to_storage(w1, dtype), G1


def update_rows_master(master: np.ndarray, G: np.ndarray | None, g: np.ndarray, opt: str,
                       lr: float, eps: float, dtype: str):
    """One optimizer step on touched rows of a table kept as an fp32 master
    plus a low-precision copy (GTC 2022 deck, slide "WEIGHT CONVERSION FOR
    MIXED PRECISION TRAINING"): the fp32 step runs on the master, and the copy
    is the master rounded to the storage type (RNE). Returns
    (master', copy', G'), the copy widened to fp32."""
    m32 = np.asarray(master, dtype=np.float32)
    if opt == "sgd":
        m1, G1 = sgd_step(m32, g, lr), G
    elif opt == "adagrad":
        if G is None:
            raise ValueError("adagrad needs its accumulator")
        m1, G1 = adagrad_step(m32, G, g, lr, eps)
    else:
        raise ValueError(opt)
    return m1, to_storage(m1, dtype), G1


# ---------------------------------------------------------------------------
# Routing unique keys (and reduced gradients) to their owning shards
# ---------------------------------------------------------------------------

SHARD_TABLE = 0        # every row of the table on shard `shard`
SHARD_ROW_CYCLIC = 1   # row r on shard (r + shard) mod S
SHARD_ROW_BLOCK = 2    # row r on shard floor(r / ceil(rows / S))


def shard_of_keys(keys: np.ndarray, row_offset: np.ndarray, rules, S: int) -> np.ndarray:
    """Owner shard of each global key. rules[t] = (kind, shard) for table t;
    row_offset has T+1 entries (the last one is the total row count)."""
    keys = np.asarray(keys, dtype=np.int64)
    ro = np.asarray(row_offset, dtype=np.int64)
    t = np.searchsorted(ro, keys, side="right") - 1
    r = keys - ro[t]
    dest = np.empty(len(keys), dtype=np.int64)
    for tt in np.unique(t):
        sel = t == tt
        kind, shard = rules[int(tt)]
        rows = int(ro[tt + 1] - ro[tt])
        if kind == SHARD_TABLE:
            dest[sel] = shard
        elif kind == SHARD_ROW_CYCLIC:
            dest[sel] = (r[sel] + shard) % S
        elif kind == SHARD_ROW_BLOCK:
            block = -(-rows // S)
            dest[sel] = r[sel] // block
        else:
            raise ValueError(kind)
    return dest


def pack_by_shard(unique_keys: np.ndarray, row_offset: np.ndarray, rules, S: int,
                  reduced_grad: np.ndarray | None = None):
    """Group the unique keys by owner shard (a stable sort by destination, so
    keys stay ascending inside each group). Keys at or past the total row
    count (the invalid-index sentinel) are sent nowhere. Returns
    (send_keys, send_offsets[S+1], slot_of_unique, send_grad): the keys of
    shard s are send_keys[send_offsets[s]:send_offsets[s+1]], unique key u
    sits at slot_of_unique[u] (-1 if sent nowhere), send_grad[slot] is its
    reduced gradient row."""
    u = np.asarray(unique_keys, dtype=np.int64)
    total = int(np.asarray(row_offset)[-1])
    valid = np.nonzero(u < total)[0]
    dest = shard_of_keys(u[valid], row_offset, rules, S)
    order = valid[np.argsort(dest, kind="stable")]
    counts = np.bincount(dest, minlength=S)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    slot = np.full(len(u), -1, dtype=np.int64)
    slot[order] = np.arange(len(order))
    send_grad = None if reduced_grad is None else np.asarray(reduced_grad)[order]
    return u[order], offsets, slot, send_grad


# ---------------------------------------------------------------------------
# Hash-keyed lookup: 64-bit ids -> rows, handed out on first sight
# ---------------------------------------------------------------------------

class HashTables:
    """Per-table id -> row maps (plain dicts). rows[t] is table t's capacity."""

    def __init__(self, rows):
        self.rows = [int(r) for r in rows]
        self.maps = [dict() for _ in self.rows]
        self.next_free = [0] * len(self.rows)

    def translate(self, ids, offsets, T: int, B: int, insert: bool) -> np.ndarray:
        """Rows of the N lookups (-1 = no row), walking the CSR in order."""
        ids = np.asarray(ids, dtype=np.int64)
        offsets = np.asarray(offsets, dtype=np.int64)
        out = np.full(len(ids), -1, dtype=np.int64)
        for t in range(T):
            m = self.maps[t]
            for p in range(int(offsets[t * B]), int(offsets[(t + 1) * B])):
                x = int(ids[p])
                if x in m:
                    out[p] = m[x]
                elif insert and self.next_free[t] < self.rows[t]:
                    m[x] = self.next_free[t]
                    self.next_free[t] += 1
                    out[p] = m[x]
        return out


def pooled_forward_hashed(tables, hash_tables: HashTables, ids, offsets, T: int, B: int, D: int,
                          pool: str) -> np.ndarray:
    """The hash lookup fused with the pooling (GTC 2022 deck, slide "HUGECTR
    EMBEDDING LAYER"), lookup only: each id's row comes from its table's map
    (no insertion), and the bags are pooled over those rows; an id without a
    row adds nothing and still counts in its bag's length (mean)."""
    rows = hash_tables.translate(ids, offsets, T, B, insert=False)
    return pooled_forward(tables, rows, offsets, T, B, D, pool, num_rows=hash_tables.rows)
