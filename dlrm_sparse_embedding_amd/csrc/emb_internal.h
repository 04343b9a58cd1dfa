// Internal declarations shared by the HIP kernels and the C-ABI host layer.
// Not part of the public interface (that is include/emb.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "emb.h"

namespace emb {

// Per-table device descriptor (weights / Adagrad state / fp32 master per
// column slice; state and master pointers are null when absent).
struct DevTable {
  void* w[EMB_MAX_SLICES];
  float* g[EMB_MAX_SLICES];
  float* m[EMB_MAX_SLICES];
};

// Hash map of one table (hash-keyed lookup): slots [base, base + mask + 1)
// of the context's key / value / scratch arrays; rows = the table's rows.
struct HashMeta {
  long long base;
  uint32_t mask;
  int rows;
};

// Device view of the attached hash maps (caller memory).
struct HashView {
  const HashMeta* meta;       // [T] (context-owned device copy)
  unsigned long long* keys;   // [slots] id, or the free marker
  int* vals;                  // [slots] row of the id
  int* next_free;             // [T] rows handed out so far
  long long slots;
};

// Workspace of one translation of N lookups.
struct HashScratch {
  int* slot_of_pos;           // [N]
  unsigned long long* pkeys;  // [2N] pending map (new ids of the step)
  int* paux;                  // [2N]
  int* pval;                  // [2N]
  uint32_t* blk;              // [N / 2048 + 2]
  int* rank_base;             // [T + 1]
};

// Update-kernel type code: the storage type, or'ed with kMasterBit when the
// table is stepped from an fp32 master and the storage holds its RNE copy.
constexpr int kMasterBit = 8;

// Upper bound on tables per context: the row-offset array is staged in LDS
// by the update kernels (4 bytes per entry).
constexpr int kMaxTables = 4096;

// Scratch of the translation that allocates nothing: a fixed device array per
// GPU (k_hash.hip), enough for about 1.8 M lookups.
constexpr size_t kHashNoAllocBytes = 64ull << 20;
constexpr int kMaxDevices = 64;

// Segment chunking of the sorted lookups (see the reduce kernels): every
// segment is cut at multiples of kChunk sorted positions (level-0 tiles);
// partial sums of segments longer than a tile are combined per level-1 tile
// of kChunk * kL1Tiles positions, then per segment.
constexpr int kChunk = 128;
constexpr int kL1Tiles = 32;
constexpr int kChunk1 = kChunk * kL1Tiles;  // 4096 positions

// Radix sort / run-length tiles.
constexpr int kSortThreads = 256;
constexpr int kSortIPT = 8;
constexpr int kSortTile = kSortThreads * kSortIPT;  // 2048 items
constexpr int kRadixMaxBits = 10;
constexpr int kRadixMax = 1 << kRadixMaxBits;
// The table-segmented sort handles at most this many tables (every block
// rebuilds the segment map in LDS).
constexpr int kSegMaxTables = 256;

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
inline int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}
inline int round_up8(int x) { return (x + 7) & ~7; }
// Column blocks of a row of D fp32 columns at 4 columns per lane, lpr lanes.
inline unsigned col_blocks(int D, int lpr) { return (unsigned)((D + 4 * lpr - 1) / (4 * lpr)); }

// Geometry common to every table of a context.
struct Geom {
  int T;
  int D;          // logical row width
  int Dsl;        // width of one column slice
  int nslices;
  int dtype;      // EMB_F32 / EMB_BF16 / EMB_F16
  bool master;    // fp32 master weights present (low-precision storage only)
  uint32_t total_rows;
  int key_bits;   // bits needed for keys 0..total_rows (total_rows = invalid-index sentinel)
  int row_bits;   // bits needed for rows 0..max_rows (max over tables; max_rows itself
                  // stands for a key outside the table in the table-segmented sort)
};

// Device-side context block.
struct DevCtx {
  const DevTable* tables;     // [T]
  const uint32_t* row_off;    // [T+1]
  int* err_flag;              // set to 1 by kernels that see an out-of-range index
};

// Workspace carve-up for the backward / update pair.
struct WsLayout {
  size_t keys_a, keys_b;        // uint64 [N] (key << 32 | bag), ping-pong
  size_t key_of_pos;            // uint32 [N] key of each lookup in input order (total_rows + t: table t's sentinel)
  size_t seg_of_key;            // int32 [total_rows + T] segment of each key present (multi-hot inverse)
  size_t unit_grp;              // int32 [ceil(T*B/64)] 1 if each of a key-build group's 64 bags is [b, b+1)
  size_t sorted_bag;            // int32 [N] bag of each sorted lookup
  size_t inv_len;               // fp32 [T*B] 1/L per bag (mean pooling)
  size_t seg_off;               // int32 [N+1]
  size_t desc;                  // int32x4 [N + ntiles + 4] chunk descriptors (3 of slack for a scalar prefetch)
  size_t chunk_seg;             // int32 [N + ntiles] segment of each chunk
  size_t tile_first_seg;        // int32 [ntiles] segment of a tile's first position
  size_t tile_last_seg;         // int32 [ntiles] segment of a tile's last position
  size_t partial0;              // fp32 [2*ntiles][D]
  size_t partial1;              // fp32 [2*ntiles1][D]
  size_t seg_start;             // int32 [T] first position of each table's bags
  size_t ghist;                 // uint32 [digits][nblk] of a sort plan (ghist_cap entries)
  size_t segbase;               // uint32 [S+1][digits] (segbase_cap entries)
  size_t ghist_cap, segbase_cap;
  size_t rle_blk;               // uint32x4 [nblk_rle]
  size_t scalars;               // int32 [16]: [0] num_chunks
  size_t total;
  int ntiles, ntiles1, nblk_sort, nblk_rle;
};
WsLayout ws_layout(const Geom& g, long long N, int B);

// ---- launchers (defined in the .hip files) -------------------------------
// Each returns hipSuccess or the launch error. `kid` callbacks for timing are
// handled by the host layer around these calls.

hipError_t launch_init_slice(const Geom& g, const DevCtx& dc, int t, int s, int64_t rows, void* w,
                             float* state, float* master, uint64_t seed, hipStream_t st);

// max_blocks > 0 caps the grid (the kernel strides over the rest). flat
// (optional): pool from a compact [flat_rows][D] buffer of the storage type
// instead of the tables, with int32 indices into it (the unique-first forward).
hipError_t launch_forward(const Geom& g, const DevCtx& dc, const void* indices, const void* offsets,
                          int itype, long long N, int B, int pool, float* out, int max_blocks,
                          hipStream_t st, const void* flat = nullptr, long long flat_rows = 0,
                          const HashView* hash = nullptr);
// rows[u] = logical row of unique key u (storage type), u < min(*num_unique, cap)
hipError_t launch_gather_unique(const Geom& g, const DevCtx& dc, const uint32_t* ukeys,
                                const int32_t* num_unique, int cap, void* rows, hipStream_t st);

hipError_t launch_keys(const Geom& g, const DevCtx& dc, const void* indices, const void* offsets,
                       int itype, long long N, int B, int pool, const WsLayout& L, char* ws,
                       hipStream_t st);

// One stable LSD radix sort of N (key << 32 | bag) words: passes over
// shift = 0, rb, 2*rb, ... < bits, each = hist, scan, scatter.
struct SortPlan {
  bool seg;    // table-segmented: each table's positions sorted on its row bits
  int bits;    // bits sorted (key bits, or row bits when seg)
  int passes;
  int rb;      // digit bits, 8..kRadixMaxBits
  int S;       // segments (T when seg, else 1)
  int ipt;     // items per thread: tiles of 256 * ipt items
  int nblk;    // tiles of the hist / scatter grids (multiple of 8)
};
// sorts of at least this many items use 4096-item tiles
constexpr long long kSortBigN = 16ll << 20;
SortPlan sort_plan_global(int bits, long long N);
SortPlan sort_plan_dedup(const Geom& g, long long N);
struct SortBufs {
  uint32_t* ghist;            // nblk << rb entries used
  uint32_t* segbase;          // (S + 1) << rb entries used
  const int32_t* seg_start;   // [T] (table-segmented plans)
  const uint32_t* row_off;    // [T+1]
  size_t ghist_cap;           // entries of ghist and segbase
  size_t segbase_cap;
};
hipError_t launch_sort_hist(const SortPlan& p, const SortBufs& b, const uint64_t* keys, int N, int shift,
                            hipStream_t st);
hipError_t launch_sort_scan(const SortPlan& p, const SortBufs& b, int N, hipStream_t st);
hipError_t launch_sort_scatter(const SortPlan& p, const SortBufs& b, const uint64_t* in, uint64_t* out, int N,
                               int shift, hipStream_t st);

struct RleOut {
  uint32_t* unique_keys;
  int32_t* counts;
  int32_t* inverse;
  int32_t* num_unique;
};
// ngrp: key-build groups whose one-lookup-per-bag flags decide whether the
// bag of position p is p itself (0 when N != T*B: never).
hipError_t launch_rle(const Geom& g, int B, const uint64_t* sorted, int N, int ngrp, const WsLayout& L, char* ws,
                      const RleOut& o, hipStream_t st);
// Measurement aid (k_probe.hip): probe_blocks() blocks of 8 subgroups, each
// reading `reads` random 512-byte rows; sink gets one float per block.
int probe_blocks();
hipError_t launch_probe_reads(const void* buf, uint32_t nrows, uint32_t stride, int local, int reads,
                              int row_bytes, float* sink, hipStream_t st);
hipError_t launch_probe_update(const float* src, uint32_t nsrc, float* a, float* b, uint32_t nrows, int items,
                               hipStream_t st);
hipError_t launch_set_empty(const WsLayout& L, char* ws, int32_t* num_unique, hipStream_t st);

// mode: 0 = write reduced gradient, 1 = fused SGD, 2 = fused Adagrad.
// slot (mode 0, optional): segment u's gradient goes to row slot[u] of
// grad_out (skipped if negative) instead of row u.
hipError_t launch_reduce(const Geom& g, const DevCtx& dc, int mode, int N, int B, int pool,
                         const float* dY, const WsLayout& L, const char* ws,
                         const uint32_t* unique_keys, const int32_t* num_unique, float* grad_out,
                         float lr, float eps, hipStream_t st, const int32_t* slot = nullptr);
hipError_t launch_combine(const Geom& g, const DevCtx& dc, int mode, int N, const WsLayout& L,
                          const char* ws, const uint32_t* unique_keys, float* grad_out, float lr,
                          float eps, hipStream_t st, const int32_t* slot = nullptr);

// hash-keyed lookup (k_hash.hip)
hipError_t launch_hash_clear(const HashView& h, int T, hipStream_t st);
// rows_out has the integer type `itype`
// Device address of the fixed translation scratch (kHashNoAllocBytes) on
// `device`, which must be current: looked up once per device, then cached.
hipError_t hash_noalloc_scratch(int device, void** out);
hipError_t launch_hash_translate(const HashView& h, const DevCtx& dc, int T, const long long* ids,
                                 const void* offsets, int itype, int N, int B, bool insert, const HashScratch& w,
                                 void* rows_out, hipStream_t st);

// shard routing (k_pack.hip); rules: device [T] {kind, shard}
hipError_t launch_pack_dest(const Geom& g, const DevCtx& dc, const int2* rules, int S, int N,
                            const uint32_t* ukeys, const int32_t* num_unique, uint64_t* words,
                            hipStream_t st);
hipError_t launch_pack_place(const uint64_t* sorted, const uint32_t* ukeys, const int32_t* num_unique,
                             int N, int S, uint32_t* send_keys, int32_t* slot, hipStream_t st);
hipError_t launch_pack_offsets(const uint64_t* sorted, int N, int S, int32_t* send_offsets,
                               hipStream_t st);
// zero grad[0..U) and scatter-add every lookup's scaled dY row with fp32 atomics
hipError_t launch_atomic_reduce(const Geom& g, const void* offsets, int itype, long long N, int B,
                                int pool, const float* dY, const int32_t* inverse,
                                const int32_t* num_unique, float* grad, hipStream_t st);
// opt: 1 = SGD, 2 = Adagrad; reads grad_in[u] for u < *num_unique
hipError_t launch_apply(const Geom& g, const DevCtx& dc, int mode, int N,
                        const uint32_t* unique_keys, const int32_t* num_unique,
                        const float* grad_in, float lr, float eps, hipStream_t st);

}  // namespace emb
