/*
 * emb.h -- C ABI of the MI355X pooled-embedding library (libemb.so).
 *
 * The operations are those of the embedding layer of a deep learning
 * recommendation model, as the NVIDIA Merlin / HugeCTR / EMBark pages state
 * the problem:
 *   - "Merlin HugeCTR: GPU-accelerated recommender system training and
 *     inference" (GTC 2022 deck), slide "COMMON EMBEDDING PRIMITIVES":
 *     table lookup, pooling/reduction of multi-hot features, concatenation;
 *     slide "HUGECTR EMBEDDING LAYER": lookup and in-register reduction and
 *     concatenation fused into one kernel;
 *     slide "CHALLENGES OF EMBEDDING LAYER": these primitives are memory
 *     bound, tables are sharded across GPUs (one GPU's share is what this
 *     library holds);
 *     slide "WEIGHT CONVERSION FOR MIXED PRECISION TRAINING": the optimizer
 *     computes in FP32 (optionally on FP32 master weights whose
 *     low-precision cast the lookups read).
 *   - NVIDIA Merlin blog, HugeCTR section: the features of one slot are
 *     each turned into an embedding vector and reduced to a single vector.
 *   - EMBark (RecSys'24 news article, sections on embedding clusters and 3D
 *     sharding): reduction-based and unique-based compression of embedding
 *     traffic, applied here locally as key dedup + per-key gradient
 *     reduction, and as the routing of unique keys to owner shards.
 *   - Sparse Operation Kit 2.0 article (Merlin TensorFlow plugin): dynamic
 *     embedding, i.e. ids mapped to rows as they arrive (the hash-keyed
 *     lookup below).
 *
 * Conventions for every call
 *   - All tensors are caller-owned device memory (allocated e.g. by
 *     PyTorch). The library never frees caller memory. It allocates only
 *     small per-context device arrays: the descriptor block (tables, row
 *     offsets, error flag; lazily, on first use), and when those features
 *     are used the shard rules (8 bytes per table) and the hash-map layout
 *     (16 bytes per table).
 *   - A context belongs to the HIP device that is current at its first
 *     device call (its descriptor block lives there); later calls with
 *     another device current fail with EMB_E_INVAL.
 *   - Every call that takes `hip_stream` is asynchronous on that stream
 *     (a hipStream_t passed as void*; NULL = the null stream) and performs
 *     no host synchronisation, except emb_check_device_error,
 *     emb_kernel_times, and the one-time uploads named at
 *     emb_set_shard_map and emb_hash_attach.
 *   - Return value: EMB_OK (0) or a negative EMB_E_* code; then
 *     emb_last_error() returns a message (per thread). No C++ exception
 *     crosses this interface. Argument validation happens before any HIP
 *     call, so an invalid call has no effect on the device.
 *   - Layouts:
 *       table t, slice s: row-major [rows][dim/col_slices] of the storage
 *         type; element (r, c) lives in slice c / (dim/col_slices).
 *       indices: [N] int32 or int64 row ids, each in [0, rows_t).
 *       offsets: [T*B + 1], same integer type as indices, table-major: bag
 *         (t, b) is indices[offsets[t*B+b] .. offsets[t*B+b+1]);
 *         offsets[0] = 0, non-decreasing, offsets[T*B] = N.
 *       pooled output / upstream gradient: [B][T*dim] fp32, sample-major,
 *         the T pooled vectors of a sample concatenated in table order.
 *       global key of a lookup: row_offset[t] + idx, row_offset[t] being the
 *         sum of rows of tables 0..t-1 (creation order).
 */
#ifndef EMB_H_
#define EMB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define EMB_OK            0
#define EMB_E_INVAL      (-1)  /* bad argument: null pointer, size, layout */
#define EMB_E_DTYPE      (-2)  /* unknown dtype / index type / pool / optimizer */
#define EMB_E_WORKSPACE  (-3)  /* workspace smaller than emb_backward_workspace_bytes */
#define EMB_E_HIP        (-4)  /* a HIP runtime call or launch failed */
#define EMB_E_BOUNDS     (-5)  /* a kernel saw an index outside [0, rows) */
#define EMB_E_STATE      (-6)  /* call order: update without a matching backward */

/* ---- enums ------------------------------------------------------------ */
#define EMB_F32   0   /* storage types */
#define EMB_BF16  1
#define EMB_F16   2

#define EMB_I32   0   /* index / offset integer type */
#define EMB_I64   1

#define EMB_POOL_SUM   0
#define EMB_POOL_MEAN  1

#define EMB_OPT_SGD      0
#define EMB_OPT_ADAGRAD  1

#define EMB_MAX_SLICES 4

/* One table of this GPU's share.
 *   rows        >= 1
 *   dim         >= 1; dim % col_slices == 0; the bytes of one slice row
 *               (dim/col_slices * sizeof(storage)) must be a multiple of 16;
 *               dim <= 256 (fp32) or 512 (bf16/fp16).
 *   col_slices  1..EMB_MAX_SLICES; slices are a layout of one logical table
 *               (one key stream, one dedup, one pooled output block of dim),
 *               as a column-wise shard of a table is.
 *   dtype       EMB_F32 | EMB_BF16 | EMB_F16 (the only stored copy).
 *   weights[s]  device pointer of slice s, 16-byte aligned.
 *   state[s]    device fp32 Adagrad accumulator of slice s (same shape as
 *               the weight slice), or NULL for all s if Adagrad is not used.
 *   master[s]   device fp32 master weights of slice s (same shape, 16-byte
 *               aligned), or NULL for all s. Only for EMB_BF16 / EMB_F16:
 *               the mixed-precision scheme of the "Merlin HugeCTR" GTC 2022
 *               deck, slide "WEIGHT CONVERSION FOR MIXED PRECISION TRAINING"
 *               (the optimizer keeps FP32 master weights; the weights the
 *               lookups use are their low-precision cast). With a master,
 *               the update reads the master (never weights[s]), steps it in
 *               fp32, and writes the master and weights[s] = RNE(master) in
 *               the same pass; the forward reads weights[s]. Without one,
 *               weights[s] is the only copy.
 * All tables of one context must share dim, col_slices and dtype, and all
 * or none of them carry state, and all or none a master. */
typedef struct emb_table_desc {
  int64_t rows;
  int32_t dim;
  int32_t col_slices;
  int32_t dtype;
  int32_t reserved;             /* must be 0 */
  void*   weights[EMB_MAX_SLICES];
  float*  state[EMB_MAX_SLICES];
  float*  master[EMB_MAX_SLICES];
} emb_table_desc;

typedef struct emb_ctx emb_ctx;

/* Register T tables (this GPU's share). Copies the descriptors; computes
 * row_offset. Fails with EMB_E_INVAL if T < 1, if the tables disagree in
 * dim/col_slices/dtype, if the sum of rows plus
 * num_tables is >= 2^32 - 1, or on any layout
 * rule above; EMB_E_DTYPE on an unknown dtype. Touches no device state:
 * the small device descriptor block is uploaded on the first launch. */
int emb_create_tables(const emb_table_desc* descs, int32_t num_tables, emb_ctx** out);

/* Frees the context and its descriptor block (synchronises the device
 * if the block was uploaded). NULL is a no-op. */
void emb_destroy_tables(emb_ctx* ctx);

/* Sum of rows of tables 0..t-1 for t = 0..T (T+1 values) into row_offset. */
int emb_row_offsets(const emb_ctx* ctx, int64_t* row_offset);

/* Synthetic table contents (set-up, not part of a step): every element
 * (t, r, c) becomes w = fp32(v) * fp32(0.1f * 2^-24) with
 * v = (splitmix64(seed ^ (t << 40) ^ (r*dim + c)) >> 40) - 2^23, i.e.
 * U(-0.05, 0.05), rounded to the storage type with round-to-nearest-even;
 * fp32 masters (if present) get w itself, so the stored copy is their RNE
 * cast; Adagrad state (if present) is set to 0. SplitMix64 as published by
 * Steele, Lea & Flood (OOPSLA 2014). */
int emb_init_uniform(emb_ctx* ctx, uint64_t seed, void* hip_stream);

/* Pooled forward: out[b][t*dim + c] = sum over bag (t, b) of
 * W_t[idx][c] (EMB_POOL_SUM) or that sum / bag length (EMB_POOL_MEAN),
 * accumulated in fp32 whatever the storage type; an empty bag gives 0.
 * N = number of lookups (= offsets[T*B]), B = batch size (samples).
 * A lookup whose index is outside [0, rows_t) contributes nothing, still
 * counts in its bag's length (the mean divides by offsets[b+1] - offsets[b]),
 * and raises the context's device error flag (see emb_check_device_error). */
int emb_forward_pooled(emb_ctx* ctx, const void* indices, const void* offsets,
                       int32_t itype, int64_t N, int32_t B, int32_t pool,
                       float* out, void* hip_stream);

/* Unique-first pooled forward: the unique-based compression of the EMBark
 * article (RecSys'24, embedding clusters) on the forward side. Needs the
 * dedup of the same lookups done ahead by emb_backward_dedup on this context
 * (same indices, offsets, itype, N, B, pool and ws); it reads that dedup's
 * unique keys, count and inverse. Each unique row is gathered once into
 * rows_buf (capacity N rows of dim elements of the storage type, 16-byte
 * aligned, rows_buf_bytes >= N * dim * sizeof(storage)), then every bag is
 * pooled from rows_buf through the inverse. out is bit-identical to
 * emb_forward_pooled's (the same rows are added in the same order). The dedup
 * stays valid for the backward that follows. EMB_E_STATE without a matching
 * dedup, EMB_E_WORKSPACE if rows_buf is too small. */
int emb_forward_pooled_unique(emb_ctx* ctx, const void* indices, const void* offsets,
                              int32_t itype, int64_t N, int32_t B, int32_t pool, const void* ws,
                              void* rows_buf, size_t rows_buf_bytes, float* out,
                              void* hip_stream);

/* Bytes of workspace emb_backward_unique_reduce needs for N lookups and
 * batch B (0 on invalid arguments). It grows with N and holds 4 bytes per
 * table row besides (a key -> unique-index map for the inverse). */
size_t emb_backward_workspace_bytes(const emb_ctx* ctx, int64_t N, int32_t B);

/* Backward, dedup part (EMBark's unique/reduction-based step, locally):
 *   global keys g_i = row_offset[t(i)] + idx_i are sorted stably (device
 *   LSD radix sort over (key, bag) pairs) and run-length encoded:
 *   unique_keys[u]  (capacity N) distinct keys, strictly ascending;
 *   counts[u]       (capacity N) multiplicity of unique_keys[u];
 *   inverse[i]      ([N]) index u of lookup i's key;
 *   *num_unique     (device int32) U, the number of distinct keys.
 *   Entries beyond U are left unspecified. If reduced_grad is not NULL
 *   (capacity N x dim fp32), reduced_grad[u] = sum over lookups of key u
 *   of scale_i * dY[b(i)][t(i)*dim ...], scale_i = 1 (sum) or 1/L (mean),
 *   accumulated in fp32 in a fixed (deterministic) order.
 * dY is [B][T*dim] fp32. ws (device, >= emb_backward_workspace_bytes)
 * carries the sorted segments to emb_sparse_update; it, offsets and dY
 * must stay valid and unchanged until that call. A lookup with an
 * out-of-range index gets the key sum(rows), which is never applied by the
 * update, and raises the device error flag. That key sorts after every
 * in-range key of the lookup's own table; when the library sorts each
 * table's lookups on their row bits (it does so whenever that takes fewer
 * radix passes than sorting the whole key), it therefore appears once per
 * table holding such lookups and unique_keys is ascending apart from it.
 * In-range keys, their counts and inverse entries are unaffected. Offsets
 * that break the CSR contract raise the flag too (see
 * emb_check_device_error).
 * N must be < 2^31. */
int emb_backward_unique_reduce(emb_ctx* ctx, const void* indices, const void* offsets,
                               int32_t itype, int64_t N, int32_t B, int32_t pool,
                               const float* dY, void* ws, size_t ws_bytes,
                               uint32_t* unique_keys, int32_t* counts, int32_t* inverse,
                               int32_t* num_unique, float* reduced_grad, void* hip_stream);

/* The dedup half of emb_backward_unique_reduce alone: global keys, sort,
 * run-length encoding -> unique_keys, counts, inverse, *num_unique and the
 * sorted segments in ws (same outputs, same layouts). It needs the batch's
 * indices and offsets but not dY, so a caller may run it early -- e.g. on a
 * second stream concurrently with emb_forward_pooled, the way EMBark dedups
 * a batch's keys (unique-based compression) before the exchange. The next
 * emb_backward_unique_reduce on this context with the same indices, offsets,
 * itype, N, B, pool, ws and output buffers then skips its own dedup; a
 * backward on the same ws with other arguments discards it. Dedups into
 * different workspaces may be pending together (up to 8; a ninth replaces
 * the oldest), so a caller can run several batches ahead. A dedup into the
 * ws of the last backward cancels that backward for emb_sparse_update. The
 * caller orders the calls (same stream or an event) and keeps the buffers
 * unchanged in between. */
int emb_backward_dedup(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype,
                       int64_t N, int32_t B, int32_t pool, void* ws, size_t ws_bytes,
                       uint32_t* unique_keys, int32_t* counts, int32_t* inverse,
                       int32_t* num_unique, void* hip_stream);

/* Sparse optimizer step on the rows the last backward (with this ws) found,
 * in place, each unique row read and written exactly once:
 *   SGD:     w <- w - (lr*g)
 *   Adagrad: G <- G + g*g;  w <- w - (lr*g) / (sqrt(G) + eps)
 * in fp32 with each operation rounded separately in this order, then w
 * rounded to the storage type with round-to-nearest-even. With fp32
 * masters, w is the master (the stored copy is not read) and the master and
 * its RNE cast are both written in the same pass. g is
 * reduced_grad[u] if reduced_grad is not NULL (the buffer the backward
 * filled), else it is reduced from dY inside the update kernel (fused
 * path, no materialised gradient). Rows no lookup touched are not read or
 * written. EMB_E_STATE if ws is not the workspace of this context's last
 * backward; EMB_E_INVAL for Adagrad on tables without state, for a NULL
 * dY on the fused path, or for dY / reduced_grad not 16-byte aligned. */
int emb_sparse_update(emb_ctx* ctx, int32_t opt, float lr, float eps,
                      const void* ws, const float* dY, const float* reduced_grad,
                      void* hip_stream);

/* Evidence variant of the gradient reduction (atomics instead of sorted
 * segments), for measuring the two against each other: zeroes
 * reduced_grad[0..U) and adds scale_i * dY[b(i)][t(i)*dim ...] into
 * reduced_grad[inverse[i]] for every lookup with fp32 atomic adds, one
 * subgroup per bag (the bag's dY row is read once). inverse and num_unique
 * come from a preceding dedup of the same batch. The result equals the
 * sorted path's reduced_grad up to fp32 summation order, which here is not
 * deterministic. emb_sparse_update with this reduced_grad applies it. */
int emb_backward_atomic_reduce(emb_ctx* ctx, const void* offsets, int32_t itype, int64_t N,
                               int32_t B, int32_t pool, const float* dY, const int32_t* inverse,
                               const int32_t* num_unique, float* reduced_grad, void* hip_stream);

/* ---- routing to shards (the step before an embedding exchange) -------- */
/* EMBark (RecSys'24 article, embedding clusters and 3D sharding): tables are
 * split into shards owned by different GPUs, and the reduction-based (RB) and
 * unique-based (UB) clusters send each distinct key, and its reduced
 * gradient, once per step. The two calls below are that step for one GPU's
 * share: they route the unique keys of the last backward to their owner
 * shards and lay them out (and, for RB, the reduced gradients) grouped by
 * destination, ready for an all-to-all. Nothing here talks to another GPU. */
#define EMB_SHARD_TABLE       0   /* every row of the table on shard `shard` */
#define EMB_SHARD_ROW_CYCLIC  1   /* row r on shard (r + shard) mod S */
#define EMB_SHARD_ROW_BLOCK   2   /* row r on shard r / ceil(rows / S); shard = 0 */
#define EMB_MAX_SHARDS        4096

typedef struct emb_shard_rule {
  int32_t kind;    /* EMB_SHARD_* */
  int32_t shard;   /* see kind; 0 <= shard < S */
} emb_shard_rule;

/* Sets the owner rule of every table (rules[T], host memory, copied) and the
 * shard count S (1..EMB_MAX_SHARDS). EMB_E_INVAL on a bad rule. The first
 * emb_pack_by_shard after this call uploads the rules (8 bytes per table) to
 * a device array the context owns, with a synchronous copy. */
int emb_set_shard_map(emb_ctx* ctx, const emb_shard_rule* rules, int32_t num_shards);

/* Groups the unique keys of this context's last backward (the call that
 * filled `ws`, with N lookups) by owner shard: a stable sort by destination,
 * so keys stay ascending inside a shard. Outputs (device, caller-owned):
 *   send_keys[N]         the keys of shard s at
 *                        [send_offsets[s], send_offsets[s+1])
 *   send_offsets[S+1]    send_offsets[S] = number of keys sent
 *   slot_of_unique[N]    unique key u sits at send_keys[slot_of_unique[u]];
 *                        -1 for the invalid-index sentinel key (sent nowhere)
 *   send_grad[N][dim]    RB only (dY != NULL): the reduced gradient of the key
 *                        at each slot, reduced straight into its slot (the
 *                        same values, bit for bit, as emb_backward_unique_reduce
 *                        writes in unique-key order); NULL for keys only (UB).
 * Entries past send_offsets[S] are unspecified. Uses the sort buffers of `ws`
 * as scratch and leaves the segment data intact, so emb_sparse_update can still
 * follow. EMB_E_STATE if ws is not the last backward's workspace or no shard
 * map is set; EMB_E_INVAL on NULL / misaligned buffers (send_grad and dY are
 * given together or not at all). */
int emb_pack_by_shard(emb_ctx* ctx, void* ws, const float* dY, uint32_t* send_keys,
                      int32_t* send_offsets, int32_t* slot_of_unique, float* send_grad,
                      void* hip_stream);

/* ---- hash-keyed lookup (feature ids -> rows) ----------------------------- */
/* "Merlin HugeCTR" GTC 2022 deck, slide "HUGECTR EMBEDDING LAYER": a GPU
 * hash table lookup fused with the pooling; the dynamic embedding of the
 * Sparse Operation Kit 2.0 article. Lookups carry arbitrary int64 ids (every
 * value but INT64_MIN, which marks a free slot); each table keeps a device
 * hash map from id to one of its rows. With insertion, an id a table has not
 * seen gets the table's next free row, ids taken in order of first appearance
 * in the CSR (so the id -> row mapping is deterministic); once a table's rows
 * are used up, new ids get no row (rows are never freed). The maps live in
 * caller memory: one region of emb_hash_bytes bytes, 2^k slots per table (at
 * least twice its rows, 12 bytes per slot) plus a counter per table; only ids
 * holding a row are stored. */

/* Bytes of map memory for this context's tables (0 if the slots would not
 * fit int32 indices or a table has 2^31 - 1 rows or more). */
size_t emb_hash_bytes(const emb_ctx* ctx);

/* Attaches the map memory (device, 256-byte aligned, >= emb_hash_bytes) and
 * empties every map on hip_stream. Uploads the per-table map layout (16 bytes
 * per table) to a device array the context owns, with a synchronous copy. */
int emb_hash_attach(emb_ctx* ctx, void* mem, size_t bytes, void* hip_stream);

/* Scratch bytes emb_hash_translate needs for N lookups. */
size_t emb_hash_workspace_bytes(const emb_ctx* ctx, int64_t N);

/* ids[N] (int64) -> rows_out[N] (row within the table of each lookup's bag,
 * -1 for an id without a row), rows_out of the integer type of offsets
 * (itype), so that rows_out and offsets feed emb_forward_pooled and the
 * backward directly (a -1 row counts as an out-of-range index there).
 * insert != 0 hands out rows to new ids as described above; insert == 0 only
 * looks up. offsets as for emb_forward_pooled; ws holds the step's pending
 * map of new ids (emb_hash_workspace_bytes: about 36 bytes per lookup).
 * Raises bit 4 of the device flag (EMB_E_INVAL from emb_check_device_error)
 * for an id equal to INT64_MIN. EMB_E_STATE if no map memory is attached. */
int emb_hash_translate(emb_ctx* ctx, const int64_t* ids, const void* offsets, int32_t itype,
                       int64_t N, int32_t B, int32_t insert, void* ws, size_t ws_bytes,
                       void* rows_out, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * translation as emb_hash_translate, same arguments and results, with its
 * scratch in a fixed 64 MiB device array the library holds on every GPU it
 * runs on (until the process ends) instead of a caller workspace. Allocates
 * nothing and records no timing events. N is limited to what fits:
 * emb_hash_workspace_bytes(ctx, N) <= 64 MiB (about 1.8 M lookups), else
 * EMB_E_WORKSPACE. The array is shared by every call on one GPU and keeps the
 * last call's contents (each call clears what it needs), so calls that
 * overlap on one GPU -- on two streams, or from two threads -- race and give
 * undefined results; order them. EMB_E_STATE if no map memory is attached;
 * EMB_E_INVAL if the current device is not the context's. */
int emb_hash_translate_noalloc(emb_ctx* ctx, const int64_t* ids, const void* offsets, int32_t itype,
                               int64_t N, int32_t B, int32_t insert, void* rows_out, void* hip_stream);

/* Fused hash lookup + pooled forward (lookup only, no insertion): as
 * emb_forward_pooled with each lookup's row found in its table's map; an id
 * without a row contributes nothing (no error) and still counts in its bag's
 * length under EMB_POOL_MEAN. EMB_E_STATE if no map memory is attached. */
int emb_forward_pooled_hashed(emb_ctx* ctx, const int64_t* ids, const void* offsets, int32_t itype,
                              int64_t N, int32_t B, int32_t pool, float* out, void* hip_stream);

/* Copies the number of rows handed out per table (int32[T], device) into
 * used, on hip_stream. */
int emb_hash_rows_used(emb_ctx* ctx, int32_t* used, void* hip_stream);

/* Message of the last failed call on this thread ("" if none). */
const char* emb_last_error(void);

/* Synchronises hip_stream, then reports (and clears) what the kernels of
 * this context flagged since the last check: EMB_E_BOUNDS if one saw an
 * index outside [0, rows_t); else EMB_E_INVAL if the backward's key build
 * saw offsets that break the CSR contract above (offsets[0] != 0, a
 * decreasing step, or offsets[T*B] != N), or the id translation saw the
 * reserved id INT64_MIN; else EMB_OK. Malformed offsets
 * never make a kernel access memory outside the caller's buffers: every
 * kernel clamps offsets into [0, N], and the key build still gives every
 * position in [0, N) an in-range key or the never-applied sentinel, but the
 * results of such a call are unspecified. */
int emb_check_device_error(emb_ctx* ctx, void* hip_stream);

/* ---- measurement ------------------------------------------------------ */
/* Kernel families timed by emb_kernel_times (index into its outputs). */
#define EMB_K_INIT          0
#define EMB_K_FORWARD       1
#define EMB_K_KEYS          2
#define EMB_K_SORT_HIST     3
#define EMB_K_SORT_SCAN     4
#define EMB_K_SORT_SCATTER  5
#define EMB_K_RLE           6
#define EMB_K_REDUCE        7   /* segmented reduce (+ fused update) */
#define EMB_K_COMBINE       8   /* long-segment combine (+ update) */
#define EMB_K_APPLY         9   /* update from a materialised gradient */
#define EMB_K_ATOMIC       10   /* atomic reduction (evidence variant) */
#define EMB_K_PACK         11   /* shard routing: destinations, placement, offsets */
#define EMB_K_GATHER       12   /* unique rows into the compact buffer */
#define EMB_K_HASH         13   /* id -> row translation (and map reset) */
#define EMB_K_COUNT        14

/* enable != 0: from now on every kernel launch of this context is
 * bracketed by HIP events recorded on the launch stream. */
int emb_set_kernel_timing(emb_ctx* ctx, int32_t enable);

/* Waits for the recorded events, adds up the elapsed time (ms) and the
 * number of launches per kernel family into ms[EMB_K_COUNT] and
 * launches[EMB_K_COUNT], and forgets them. */
int emb_kernel_times(emb_ctx* ctx, double* ms, int64_t* launches);

/* Measurement aid, not part of the method (no context): the cache and HBM
 * read ceilings that the path's kernels are compared with. Launches
 * emb_probe_blocks() blocks of 256 lanes on the stream, in subgroups of
 * row_bytes / 16 lanes (256 or 512 bytes per row: 16 bytes per lane); each
 * subgroup reads `reads` rows at pseudo-random indices in [0, nrows), row r
 * starting at byte r*stride of buf. With xcd_local != 0, block b reads only
 * rows of its eighth of [0, nrows): blocks are dealt round robin to the 8
 * XCDs, so each XCD's L2 serves its own eighth. Logical bytes read:
 * emb_probe_blocks() * 256 * reads * 16 (whatever the row size). buf
 * (device, >= (nrows - 1) * stride + row_bytes bytes, 16-byte aligned) is
 * only read; sink (device, >= emb_probe_blocks() floats) receives one value
 * per block. EMB_E_INVAL for NULL or misaligned pointers, row_bytes other
 * than 256 or 512, nrows < 8 or >= 2^32, stride < row_bytes or not a
 * multiple of 16 or >= 2^32, reads not in [4, 65536] or not a multiple of 4. */
int32_t emb_probe_blocks(void);
int emb_probe_reads(const void* buf, int64_t nrows, int64_t stride, int32_t xcd_local, int32_t reads,
                    int32_t row_bytes, float* sink, void* hip_stream);

/* Measurement aid, not part of the method (no context): the ceiling of the
 * fused Adagrad update's access mix, random 512-byte rows read and written.
 * Launches emb_probe_blocks() blocks of 8 subgroups of 32 lanes, grid-strided
 * over items i < items. Item i reads 3 rows of src (2 when i mod 50 >= 34)
 * at pseudo-random indices in [0, nsrc) and the row r of a and of b at one
 * pseudo-random r in [0, nrows), then writes both rows back (a step of the
 * summed src rows). Row k of a buffer is the 128 floats at element k*128.
 * Bytes per launch: 512 * (n_src_rows + 4 * items), n_src_rows = 3 * n3 +
 * 2 * (items - n3), n3 = 34 * (items / 50) + min(items mod 50, 34). Items
 * may draw the same r; their writes race, and a and b hold meaningless
 * values afterwards (src is only read). src (device, >= nsrc * 512 bytes),
 * a and b (device, >= nrows * 512 bytes each), all 16-byte aligned.
 * EMB_E_INVAL for NULL or misaligned pointers, nsrc or nrows not in
 * [1, 2^32), items < 1. */
int emb_probe_update(const float* src, int64_t nsrc, float* a, float* b, int64_t nrows, int32_t items,
                     void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* EMB_H_ */
