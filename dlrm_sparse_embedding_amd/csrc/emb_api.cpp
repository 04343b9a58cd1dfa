// C-ABI host layer of libemb.so: argument validation, context / descriptor
// management, workspace carve-up, kernel sequencing on the caller's stream,
// optional per-kernel HIP-event timing. No C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "emb.h"
#include "emb_internal.h"

using namespace emb;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return EMB_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(EMB_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct TimedLaunch {
  int kid;
  hipEvent_t e0, e1;
};

}  // namespace

struct emb_ctx {
  std::vector<emb_table_desc> desc;
  std::vector<int64_t> row_off;  // T+1
  Geom g{};
  bool has_state = false;
  // device block (lazily uploaded)
  int device = -1;
  void* dev_block = nullptr;
  DevCtx dc{};
  // last backward, consumed by emb_sparse_update
  struct {
    const void* ws = nullptr;
    const void* offsets = nullptr;
    int itype = 0;
    long long N = 0;
    int B = 0;
    int pool = 0;
    const uint32_t* unique_keys = nullptr;
    const int32_t* num_unique = nullptr;
    bool valid = false;
  } last;
  // dedups done ahead by emb_backward_dedup, one per workspace (at most
  // kPendingDedups at once), each consumed by the next backward on its
  // workspace
  struct DedupRec {
    const void* indices = nullptr;
    const void* offsets = nullptr;
    int itype = 0;
    long long N = 0;
    int B = 0;
    int pool = 0;
    const void* ws = nullptr;
    const uint32_t* unique_keys = nullptr;
    const int32_t* counts = nullptr;
    const int32_t* inverse = nullptr;
    const int32_t* num_unique = nullptr;
    bool valid = false;
    unsigned long long seq = 0;  // issue order, to replace the oldest when all are taken
  };
  DedupRec dedup[8];
  unsigned long long dedup_seq = 0;
  // shard map (emb_set_shard_map): host copy, device copy uploaded on first use
  std::vector<emb_shard_rule> shard_rules;
  int num_shards = 0;
  void* dev_rules = nullptr;
  bool rules_dirty = false;
  // hash maps (emb_hash_attach)
  void* dev_hmeta = nullptr;
  HashView hv{};
  bool hash_ready = false;
  // timing
  bool timing = false;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> free_events;
};

namespace {
// The dedup done ahead into ws, or null.
const emb_ctx::DedupRec* find_dedup(const emb_ctx* c, const void* ws) {
  for (const auto& d : c->dedup)
    if (d.valid && d.ws == ws) return &d;
  return nullptr;
}
}  // namespace

namespace {

int ensure_device(emb_ctx* c) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (c->dev_block) {
    if (dev != c->device)
      return fail(EMB_E_INVAL, "the context lives on device %d but device %d is current", c->device, dev);
    return EMB_OK;
  }
  const int T = c->g.T;
  const size_t tab_bytes = sizeof(DevTable) * (size_t)T;
  const size_t ro_off = (tab_bytes + 255) & ~size_t(255);
  const size_t ro_bytes = sizeof(uint32_t) * (size_t)(T + 1);
  const size_t err_off = (ro_off + ro_bytes + 255) & ~size_t(255);
  const size_t total = err_off + 256;
  std::vector<char> host(total, 0);
  DevTable* ht = reinterpret_cast<DevTable*>(host.data());
  for (int t = 0; t < T; ++t) {
    for (int s = 0; s < EMB_MAX_SLICES; ++s) {
      ht[t].w[s] = c->desc[t].weights[s];
      ht[t].g[s] = c->desc[t].state[s];
      ht[t].m[s] = c->desc[t].master[s];
    }
  }
  uint32_t* hro = reinterpret_cast<uint32_t*>(host.data() + ro_off);
  for (int t = 0; t <= T; ++t) hro[t] = (uint32_t)c->row_off[t];
  void* p = nullptr;
  e = hipMalloc(&p, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(descriptor block)");
  e = hipMemcpy(p, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(e, "hipMemcpy(descriptor block)");
  }
  c->dev_block = p;
  c->device = dev;
  c->dc.tables = reinterpret_cast<const DevTable*>(p);
  c->dc.row_off = reinterpret_cast<const uint32_t*>(static_cast<char*>(p) + ro_off);
  c->dc.err_flag = reinterpret_cast<int*>(static_cast<char*>(p) + err_off);
  return EMB_OK;
}

hipEvent_t take_event(emb_ctx* c) {
  if (!c->free_events.empty()) {
    hipEvent_t e = c->free_events.back();
    c->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with events when timing is on.
struct KScope {
  emb_ctx* c;
  int kid;
  hipStream_t st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  KScope(emb_ctx* c_, int kid_, hipStream_t st_) : c(c_), kid(kid_), st(st_) {
    if (c->timing) {
      e0 = take_event(c);
      e1 = take_event(c);
      if (e0) (void)hipEventRecord(e0, st);
    }
  }
  ~KScope() {
    if (e0 && e1) {
      (void)hipEventRecord(e1, st);
      c->pending.push_back({kid, e0, e1});
    } else {  // an event could not be created: time nothing, keep the other one
      if (e0) c->free_events.push_back(e0);
      if (e1) c->free_events.push_back(e1);
    }
  }
};

int dtype_bytes(int dt) { return dt == EMB_F32 ? 4 : 2; }

int check_itype(int itype) {
  if (itype != EMB_I32 && itype != EMB_I64) return fail(EMB_E_DTYPE, "itype %d is not EMB_I32/EMB_I64", itype);
  return EMB_OK;
}

int check_pool(int pool) {
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return fail(EMB_E_DTYPE, "pool %d is not SUM/MEAN", pool);
  return EMB_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

namespace emb {

WsLayout ws_layout(const Geom& g, long long N, int B) {
  WsLayout L{};
  const long long TB = (long long)g.T * B;
  L.ntiles = (int)((N + kChunk - 1) / kChunk);
  L.ntiles1 = (int)((N + kChunk1 - 1) / kChunk1);
  const SortPlan sp = sort_plan_dedup(g, N);
  L.nblk_sort = sp.nblk;
  L.nblk_rle = (int)((N + kSortTile - 1) / kSortTile);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~size_t(255);
    return o;
  };
  L.keys_a = take(8ull * N);
  L.keys_b = take(8ull * N);
  L.key_of_pos = take(4ull * N);
  L.seg_of_key = take(4ull * ((size_t)g.total_rows + (size_t)g.T));
  L.unit_grp = take(4ull * ((TB + 63) / 64 + 1));
  L.sorted_bag = take(4ull * N);
  L.inv_len = take(4ull * (TB > 0 ? TB : 1));
  L.seg_off = take(4ull * (N + 1));
  L.desc = take(16ull * (N + L.ntiles + 4));  // + 3 entries read past the end by a wave's scalar prefetch
  L.chunk_seg = take(4ull * (N + L.ntiles + 1));
  L.tile_first_seg = take(4ull * (L.ntiles > 0 ? L.ntiles : 1));
  L.tile_last_seg = take(4ull * (L.ntiles > 0 ? L.ntiles : 1));
  L.partial0 = take(4ull * 2 * (L.ntiles > 0 ? L.ntiles : 1) * g.D);
  L.partial1 = take(4ull * 2 * (L.ntiles1 > 0 ? L.ntiles1 : 1) * g.D);
  L.seg_start = take(4ull * g.T);
  // sized for the widest digit, so that any plan over these N words fits:
  // the dedup's, and the shard-routing sort's (a global plan over the same N
  // with digits up to kRadixMaxBits wide)
  L.ghist_cap = (size_t)L.nblk_sort << kRadixMaxBits;
  L.segbase_cap = (size_t)(sp.S + 1) << kRadixMaxBits;
  L.ghist = take(4ull * L.ghist_cap);
  L.segbase = take(4ull * L.segbase_cap);
  L.rle_blk = take(16ull * (L.nblk_rle > 0 ? L.nblk_rle : 1));
  L.scalars = take(64);
  L.total = off;
  return L;
}

}  // namespace emb

extern "C" {

const char* emb_last_error(void) { return g_last_error.c_str(); }

int emb_create_tables(const emb_table_desc* descs, int32_t num_tables, emb_ctx** out) {
  try {
    if (!out) return fail(EMB_E_INVAL, "out is NULL");
    *out = nullptr;
    if (!descs) return fail(EMB_E_INVAL, "descs is NULL");
    if (num_tables < 1) return fail(EMB_E_INVAL, "num_tables must be >= 1 (got %d)", num_tables);
    if (num_tables > kMaxTables) return fail(EMB_E_INVAL, "num_tables must be <= %d", kMaxTables);
    const emb_table_desc& d0 = descs[0];
    if (d0.dtype != EMB_F32 && d0.dtype != EMB_BF16 && d0.dtype != EMB_F16)
      return fail(EMB_E_DTYPE, "table 0: unknown dtype %d", d0.dtype);
    if (d0.col_slices < 1 || d0.col_slices > EMB_MAX_SLICES)
      return fail(EMB_E_INVAL, "table 0: col_slices must be in 1..%d", EMB_MAX_SLICES);
    if (d0.dim < 1 || d0.dim % d0.col_slices != 0)
      return fail(EMB_E_INVAL, "table 0: dim %d not a positive multiple of col_slices %d", d0.dim, d0.col_slices);
    const int eb = dtype_bytes(d0.dtype);
    const int Dsl = d0.dim / d0.col_slices;
    if ((Dsl * eb) % 16 != 0)
      return fail(EMB_E_INVAL, "slice row of %d bytes is not a multiple of 16", Dsl * eb);
    if (d0.dim * eb > 64 * 16)
      return fail(EMB_E_INVAL, "dim %d too wide (row bytes must be <= 1024)", d0.dim);
    const bool state0 = d0.state[0] != nullptr;
    const bool master0 = d0.master[0] != nullptr;
    if (master0 && d0.dtype == EMB_F32)
      return fail(EMB_E_INVAL, "fp32 master weights are only for bf16 / fp16 tables");
    int64_t sum = 0;
    for (int t = 0; t < num_tables; ++t) {
      const emb_table_desc& d = descs[t];
      if (d.dtype != EMB_F32 && d.dtype != EMB_BF16 && d.dtype != EMB_F16)
        return fail(EMB_E_DTYPE, "table %d: unknown dtype %d", t, d.dtype);
      if (d.dim != d0.dim || d.col_slices != d0.col_slices || d.dtype != d0.dtype)
        return fail(EMB_E_INVAL, "table %d: dim/col_slices/dtype differ from table 0", t);
      if (d.reserved != 0) return fail(EMB_E_INVAL, "table %d: reserved must be 0", t);
      if (d.rows < 1) return fail(EMB_E_INVAL, "table %d: rows must be >= 1", t);
      for (int s = 0; s < EMB_MAX_SLICES; ++s) {
        const bool used = s < d.col_slices;
        if (used && !d.weights[s]) return fail(EMB_E_INVAL, "table %d: weights[%d] is NULL", t, s);
        if (used && !aligned(d.weights[s], 16)) return fail(EMB_E_INVAL, "table %d: weights[%d] not 16-byte aligned", t, s);
        if (used && ((d.state[s] != nullptr) != state0))
          return fail(EMB_E_INVAL, "table %d: state must be given for all slices of all tables or none", t);
        if (used && d.state[s] && !aligned(d.state[s], 16))
          return fail(EMB_E_INVAL, "table %d: state[%d] not 16-byte aligned", t, s);
        if (used && ((d.master[s] != nullptr) != master0))
          return fail(EMB_E_INVAL, "table %d: master must be given for all slices of all tables or none", t);
        if (used && d.master[s] && !aligned(d.master[s], 16))
          return fail(EMB_E_INVAL, "table %d: master[%d] not 16-byte aligned", t, s);
        if (!used && (d.state[s] || d.master[s] || d.weights[s]))
          return fail(EMB_E_INVAL, "table %d: pointers of slice %d >= col_slices must be NULL", t, s);
      }
      sum += d.rows;
      if (sum + num_tables >= (int64_t)0xFFFFFFFFll)
        return fail(EMB_E_INVAL, "sum of rows plus the number of tables must be < 2^32 - 1");
    }
    emb_ctx* c = new (std::nothrow) emb_ctx();
    if (!c) return fail(EMB_E_INVAL, "out of host memory");
    c->desc.assign(descs, descs + num_tables);
    c->row_off.resize(num_tables + 1);
    c->row_off[0] = 0;
    for (int t = 0; t < num_tables; ++t) c->row_off[t + 1] = c->row_off[t] + descs[t].rows;
    c->g.T = num_tables;
    c->g.D = d0.dim;
    c->g.Dsl = Dsl;
    c->g.nslices = d0.col_slices;
    c->g.dtype = d0.dtype;
    c->g.master = master0;
    c->g.total_rows = (uint32_t)sum;
    int bits = 1;
    while (bits < 32 && (1ull << bits) <= (uint64_t)sum) ++bits;
    c->g.key_bits = bits;  // keys 0..sum (sum = invalid-index sentinel)
    int64_t max_rows = 0;
    for (int t = 0; t < num_tables; ++t) max_rows = std::max<int64_t>(max_rows, descs[t].rows);
    int rbits = 1;
    while (rbits < 32 && (1ull << rbits) <= (uint64_t)max_rows) ++rbits;
    c->g.row_bits = rbits;  // rows 0..max_rows (max_rows = a key outside its table)
    c->has_state = state0;
    *out = c;
    return ok();
  } catch (...) {
    return fail(EMB_E_INVAL, "internal error in emb_create_tables");
  }
}

void emb_destroy_tables(emb_ctx* ctx) {
  if (!ctx) return;
  if (ctx->dev_block) {
    (void)hipDeviceSynchronize();
    (void)hipFree(ctx->dev_block);
  }
  for (auto& p : ctx->pending) {
    (void)hipEventDestroy(p.e0);
    (void)hipEventDestroy(p.e1);
  }
  for (auto e : ctx->free_events) (void)hipEventDestroy(e);
  if (ctx->dev_rules) (void)hipFree(ctx->dev_rules);
  if (ctx->dev_hmeta) (void)hipFree(ctx->dev_hmeta);
  delete ctx;
}

int emb_row_offsets(const emb_ctx* ctx, int64_t* row_offset) {
  if (!ctx || !row_offset) return fail(EMB_E_INVAL, "NULL argument");
  for (int t = 0; t <= ctx->g.T; ++t) row_offset[t] = ctx->row_off[t];
  return ok();
}

int emb_init_uniform(emb_ctx* ctx, uint64_t seed, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  int rc = ensure_device(ctx);
  if (rc != EMB_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  for (int t = 0; t < ctx->g.T; ++t) {
    for (int s = 0; s < ctx->g.nslices; ++s) {
      KScope ks(ctx, EMB_K_INIT, st);
      hipError_t e = launch_init_slice(ctx->g, ctx->dc, t, s, ctx->desc[t].rows, ctx->desc[t].weights[s],
                                       ctx->desc[t].state[s], ctx->desc[t].master[s], seed, st);
      if (e != hipSuccess) return hip_fail(e, "init kernel");
    }
  }
  return ok();
}

int emb_forward_pooled(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype, int64_t N,
                       int32_t B, int32_t pool, float* out, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  int rc = check_itype(itype);
  if (rc) return rc;
  if ((rc = check_pool(pool))) return rc;
  if (B < 0 || N < 0) return fail(EMB_E_INVAL, "negative B or N");
  if (N >= (1ll << 31)) return fail(EMB_E_INVAL, "N must be < 2^31");
  if (B == 0) return N == 0 ? ok() : fail(EMB_E_INVAL, "B == 0 with N > 0");
  if (!offsets || !out) return fail(EMB_E_INVAL, "offsets/out is NULL");
  if (N > 0 && !indices) return fail(EMB_E_INVAL, "indices is NULL");
  if (!aligned(out, 16)) return fail(EMB_E_INVAL, "out must be 16-byte aligned");
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  KScope ks(ctx, EMB_K_FORWARD, st);
  hipError_t e = launch_forward(ctx->g, ctx->dc, indices, offsets, itype, N, B, pool, out,
                                0, st);
  if (e != hipSuccess) return hip_fail(e, "forward kernel");
  return ok();
}

int emb_forward_pooled_unique(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype, int64_t N,
                              int32_t B, int32_t pool, const void* ws, void* rows_buf, size_t rows_buf_bytes,
                              float* out, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  int rc = check_itype(itype);
  if (rc) return rc;
  if ((rc = check_pool(pool))) return rc;
  if (B < 0 || N < 0) return fail(EMB_E_INVAL, "negative B or N");
  if (N >= (1ll << 31)) return fail(EMB_E_INVAL, "N must be < 2^31");
  if (B == 0) return N == 0 ? ok() : fail(EMB_E_INVAL, "B == 0 with N > 0");
  if (!offsets || !out) return fail(EMB_E_INVAL, "offsets/out is NULL");
  if (!aligned(out, 16)) return fail(EMB_E_INVAL, "out must be 16-byte aligned");
  const emb_ctx::DedupRec* dp = find_dedup(ctx, ws);
  if (!(dp && dp->indices == indices && dp->offsets == offsets && dp->itype == itype && dp->N == N && dp->B == B &&
        dp->pool == pool))
    return fail(EMB_E_STATE, "no dedup of these lookups was done ahead on this context (emb_backward_dedup)");
  const emb_ctx::DedupRec& d = *dp;
  const size_t need = (size_t)N * ctx->g.D * dtype_bytes(ctx->g.dtype);
  if (N > 0 && (!rows_buf || !aligned(rows_buf, 16))) return fail(EMB_E_INVAL, "rows_buf is NULL or misaligned");
  if (rows_buf_bytes < need) return fail(EMB_E_WORKSPACE, "rows_buf of %zu bytes < %zu needed", rows_buf_bytes, need);
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  {
    KScope ks(ctx, EMB_K_GATHER, st);
    if ((e = launch_gather_unique(ctx->g, ctx->dc, d.unique_keys, d.num_unique, (int)N, rows_buf, st)) != hipSuccess)
      return hip_fail(e, "gather unique rows");
  }
  {
    KScope ks(ctx, EMB_K_FORWARD, st);
    if ((e = launch_forward(ctx->g, ctx->dc, d.inverse, offsets, itype, N, B, pool, out, 0, st,
                            rows_buf, N)) != hipSuccess)
      return hip_fail(e, "forward from unique rows");
  }
  return ok();
}

size_t emb_backward_workspace_bytes(const emb_ctx* ctx, int64_t N, int32_t B) {
  if (!ctx || N < 0 || B < 0 || N >= (1ll << 31)) return 0;
  return ws_layout(ctx->g, N, B).total;
}

}  // extern "C"

namespace {

// Argument checks shared by the dedup-only and the full backward call.
int check_dedup_args(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype, int64_t N,
                     int32_t B, int32_t pool, void* ws, size_t ws_bytes, uint32_t* unique_keys,
                     int32_t* counts, int32_t* inverse, int32_t* num_unique) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  int rc = check_itype(itype);
  if (rc) return rc;
  if ((rc = check_pool(pool))) return rc;
  if (B < 0 || N < 0) return fail(EMB_E_INVAL, "negative B or N");
  if (N >= (1ll << 31)) return fail(EMB_E_INVAL, "N must be < 2^31");
  if (B == 0 && N > 0) return fail(EMB_E_INVAL, "B == 0 with N > 0");
  if (!ws || !num_unique) return fail(EMB_E_INVAL, "ws/num_unique is NULL");
  if (N > 0 && (!indices || !offsets || !unique_keys || !counts || !inverse))
    return fail(EMB_E_INVAL, "NULL buffer");
  if (!aligned(ws, 256)) return fail(EMB_E_INVAL, "ws must be 256-byte aligned");
  if ((long long)B * ctx->g.T * ctx->g.D >= (1ll << 32))
    return fail(EMB_E_INVAL, "dY must hold fewer than 2^32 elements (B*T*dim)");
  const WsLayout L = ws_layout(ctx->g, N, B);
  if (ws_bytes < L.total)
    return fail(EMB_E_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  return EMB_OK;
}

// The passes of one radix sort of the words in *a (*b: scratch of the same
// size); on return *a holds the sorted words.
int run_sort(emb_ctx* ctx, const SortPlan& sp, const SortBufs& sb, uint64_t** a, uint64_t** b, int N,
             hipStream_t st) {
  if (((size_t)sp.nblk << sp.rb) > sb.ghist_cap || ((size_t)(sp.S + 1) << sp.rb) > sb.segbase_cap)
    return fail(EMB_E_INVAL, "internal: radix sort plan exceeds its workspace buffers");
  hipError_t e;
  for (int shift = 0; shift < sp.bits; shift += sp.rb) {
    {
      KScope ks(ctx, EMB_K_SORT_HIST, st);
      if ((e = launch_sort_hist(sp, sb, *a, N, shift, st)) != hipSuccess) return hip_fail(e, "sort histogram");
    }
    {
      KScope ks(ctx, EMB_K_SORT_SCAN, st);
      if ((e = launch_sort_scan(sp, sb, N, st)) != hipSuccess) return hip_fail(e, "sort scan");
    }
    {
      KScope ks(ctx, EMB_K_SORT_SCATTER, st);
      if ((e = launch_sort_scatter(sp, sb, *a, *b, N, shift, st)) != hipSuccess) return hip_fail(e, "sort scatter");
    }
    std::swap(*a, *b);
  }
  return EMB_OK;
}

// Keys -> radix sort -> run-length encoding, on `st`.
int run_dedup(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype, int64_t N, int32_t B,
              int32_t pool, char* w, const WsLayout& L, uint32_t* unique_keys, int32_t* counts,
              int32_t* inverse, int32_t* num_unique, hipStream_t st) {
  hipError_t e;
  if (N == 0) {
    KScope ks(ctx, EMB_K_RLE, st);
    e = launch_set_empty(L, w, num_unique, st);
    if (e != hipSuccess) return hip_fail(e, "empty backward");
    return EMB_OK;
  }
  {
    KScope ks(ctx, EMB_K_KEYS, st);
    e = launch_keys(ctx->g, ctx->dc, indices, offsets, itype, N, B, pool, L, w, st);
    if (e != hipSuccess) return hip_fail(e, "keys kernel");
  }
  uint64_t* a = reinterpret_cast<uint64_t*>(w + L.keys_a);
  uint64_t* b = reinterpret_cast<uint64_t*>(w + L.keys_b);
  const SortPlan sp = sort_plan_dedup(ctx->g, N);
  const SortBufs sb{reinterpret_cast<uint32_t*>(w + L.ghist), reinterpret_cast<uint32_t*>(w + L.segbase),
                    reinterpret_cast<const int32_t*>(w + L.seg_start), ctx->dc.row_off, L.ghist_cap,
                    L.segbase_cap};
  if (int rc = run_sort(ctx, sp, sb, &a, &b, (int)N, st)) return rc;
  {
    KScope ks(ctx, EMB_K_RLE, st);
    RleOut o{unique_keys, counts, inverse, num_unique};
    const long long TB = (long long)ctx->g.T * B;
    const int ngrp = N == TB ? (int)((TB + 63) / 64) : 0;
    if ((e = launch_rle(ctx->g, B, a, (int)N, ngrp, L, w, o, st)) != hipSuccess)
      return hip_fail(e, "run-length encode");
  }
  return EMB_OK;
}

bool same_dedup(const emb_ctx* c, const void* indices, const void* offsets, int32_t itype, int64_t N, int32_t B,
                int32_t pool, const void* ws, const uint32_t* unique_keys, const int32_t* counts,
                const int32_t* inverse, const int32_t* num_unique) {
  const emb_ctx::DedupRec* d = find_dedup(c, ws);
  return d && d->indices == indices && d->offsets == offsets && d->itype == itype && d->N == N && d->B == B &&
         d->pool == pool && d->unique_keys == unique_keys && d->counts == counts && d->inverse == inverse &&
         d->num_unique == num_unique;
}

// Forgets the dedup done ahead into ws, if any.
void drop_dedup(emb_ctx* c, const void* ws) {
  for (auto& d : c->dedup)
    if (d.valid && d.ws == ws) d.valid = false;
}

}  // namespace

extern "C" {

int emb_backward_dedup(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype, int64_t N,
                       int32_t B, int32_t pool, void* ws, size_t ws_bytes, uint32_t* unique_keys, int32_t* counts,
                       int32_t* inverse, int32_t* num_unique, void* hip_stream) {
  int rc = check_dedup_args(ctx, indices, offsets, itype, N, B, pool, ws, ws_bytes, unique_keys, counts, inverse,
                            num_unique);
  if (rc) return rc;
  if ((rc = ensure_device(ctx))) return rc;
  // this dedup overwrites ws: whatever an earlier call left there is gone
  drop_dedup(ctx, ws);
  if (ctx->last.ws == ws) ctx->last.valid = false;
  const WsLayout L = ws_layout(ctx->g, N, B);
  rc = run_dedup(ctx, indices, offsets, itype, N, B, pool, static_cast<char*>(ws), L, unique_keys, counts,
                 inverse, num_unique, static_cast<hipStream_t>(hip_stream));
  if (rc) return rc;
  // a free record, else the oldest one
  emb_ctx::DedupRec* slot = &ctx->dedup[0];
  for (auto& r : ctx->dedup) {
    if (!r.valid) {
      slot = &r;
      break;
    }
    if (r.seq < slot->seq) slot = &r;
  }
  auto& d = *slot;
  d.indices = indices;
  d.offsets = offsets;
  d.itype = itype;
  d.N = N;
  d.B = B;
  d.pool = pool;
  d.ws = ws;
  d.unique_keys = unique_keys;
  d.counts = counts;
  d.inverse = inverse;
  d.num_unique = num_unique;
  d.seq = ++ctx->dedup_seq;
  d.valid = true;
  return ok();
}

int emb_backward_unique_reduce(emb_ctx* ctx, const void* indices, const void* offsets, int32_t itype,
                               int64_t N, int32_t B, int32_t pool, const float* dY, void* ws,
                               size_t ws_bytes, uint32_t* unique_keys, int32_t* counts, int32_t* inverse,
                               int32_t* num_unique, float* reduced_grad, void* hip_stream) {
  int rc = check_dedup_args(ctx, indices, offsets, itype, N, B, pool, ws, ws_bytes, unique_keys, counts, inverse,
                            num_unique);
  if (rc) return rc;
  if (N > 0 && !dY) return fail(EMB_E_INVAL, "dY is NULL");
  if (dY && !aligned(dY, 16)) return fail(EMB_E_INVAL, "dY must be 16-byte aligned");
  if (reduced_grad && !aligned(reduced_grad, 16)) return fail(EMB_E_INVAL, "reduced_grad must be 16-byte aligned");
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* w = static_cast<char*>(ws);
  const WsLayout L = ws_layout(ctx->g, N, B);
  const bool done = same_dedup(ctx, indices, offsets, itype, N, B, pool, ws, unique_keys, counts, inverse,
                               num_unique);
  drop_dedup(ctx, ws);  // a dedup is consumed by one backward on its workspace
  ctx->last.valid = false;
  if (!done) {
    rc = run_dedup(ctx, indices, offsets, itype, N, B, pool, w, L, unique_keys, counts, inverse, num_unique, st);
    if (rc) return rc;
  }
  if (N > 0 && reduced_grad) {
    hipError_t e;
    {
      KScope ks(ctx, EMB_K_REDUCE, st);
      if ((e = launch_reduce(ctx->g, ctx->dc, 0, (int)N, B, pool, dY, L, w, unique_keys, num_unique, reduced_grad,
                             0.f, 0.f, st)) != hipSuccess)
        return hip_fail(e, "segment reduce");
    }
    {
      KScope ks(ctx, EMB_K_COMBINE, st);
      if ((e = launch_combine(ctx->g, ctx->dc, 0, (int)N, L, w, unique_keys, reduced_grad, 0.f, 0.f, st)) !=
          hipSuccess)
        return hip_fail(e, "segment combine");
    }
  }
  ctx->last.ws = ws;
  ctx->last.offsets = offsets;
  ctx->last.itype = itype;
  ctx->last.N = N;
  ctx->last.B = B;
  ctx->last.pool = pool;
  ctx->last.unique_keys = unique_keys;
  ctx->last.num_unique = num_unique;
  ctx->last.valid = true;
  return ok();
}

int emb_sparse_update(emb_ctx* ctx, int32_t opt, float lr, float eps, const void* ws, const float* dY,
                      const float* reduced_grad, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  if (opt != EMB_OPT_SGD && opt != EMB_OPT_ADAGRAD) return fail(EMB_E_DTYPE, "opt %d is not SGD/ADAGRAD", opt);
  if (opt == EMB_OPT_ADAGRAD && !ctx->has_state) return fail(EMB_E_INVAL, "Adagrad requested but the tables have no state");
  if (!ctx->last.valid || ws != ctx->last.ws)
    return fail(EMB_E_STATE, "ws is not the workspace of this context's last backward");
  const long long N = ctx->last.N;
  if (N > 0 && !reduced_grad && !dY) return fail(EMB_E_INVAL, "dY is NULL (needed by the fused path)");
  if (dY && !aligned(dY, 16)) return fail(EMB_E_INVAL, "dY must be 16-byte aligned");
  if (reduced_grad && !aligned(reduced_grad, 16)) return fail(EMB_E_INVAL, "reduced_grad must be 16-byte aligned");
  if (N == 0) return ok();
  int rc;
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const WsLayout L = ws_layout(ctx->g, N, ctx->last.B);
  const char* w = static_cast<const char*>(ws);
  const int mode = opt == EMB_OPT_SGD ? 1 : 2;
  hipError_t e;
  if (reduced_grad) {
    KScope ks(ctx, EMB_K_APPLY, st);
    if ((e = launch_apply(ctx->g, ctx->dc, mode, (int)N, ctx->last.unique_keys, ctx->last.num_unique, reduced_grad,
                          lr, eps, st)) != hipSuccess)
      return hip_fail(e, "apply update");
  } else {
    {
      KScope ks(ctx, EMB_K_REDUCE, st);
      if ((e = launch_reduce(ctx->g, ctx->dc, mode, (int)N, ctx->last.B, ctx->last.pool, dY, L, w,
                             ctx->last.unique_keys, ctx->last.num_unique, nullptr, lr, eps, st)) != hipSuccess)
        return hip_fail(e, "fused reduce + update");
    }
    {
      KScope ks(ctx, EMB_K_COMBINE, st);
      if ((e = launch_combine(ctx->g, ctx->dc, mode, (int)N, L, w, ctx->last.unique_keys, nullptr, lr, eps, st)) !=
          hipSuccess)
        return hip_fail(e, "fused combine + update");
    }
  }
  return ok();
}

int emb_backward_atomic_reduce(emb_ctx* ctx, const void* offsets, int32_t itype, int64_t N, int32_t B,
                               int32_t pool, const float* dY, const int32_t* inverse, const int32_t* num_unique,
                               float* reduced_grad, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  int rc = check_itype(itype);
  if (rc) return rc;
  if ((rc = check_pool(pool))) return rc;
  if (B < 0 || N < 0) return fail(EMB_E_INVAL, "negative B or N");
  if (N >= (1ll << 31)) return fail(EMB_E_INVAL, "N must be < 2^31");
  if (B == 0 && N > 0) return fail(EMB_E_INVAL, "B == 0 with N > 0");
  if (!num_unique || !reduced_grad) return fail(EMB_E_INVAL, "num_unique/reduced_grad is NULL");
  if (N > 0 && (!offsets || !dY || !inverse)) return fail(EMB_E_INVAL, "NULL buffer");
  if (!aligned(reduced_grad, 16) || (dY && !aligned(dY, 16)))
    return fail(EMB_E_INVAL, "dY/reduced_grad must be 16-byte aligned");
  if ((long long)B * ctx->g.T * ctx->g.D >= (1ll << 32))
    return fail(EMB_E_INVAL, "dY must hold fewer than 2^32 elements (B*T*dim)");
  if (N == 0) return ok();
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  KScope ks(ctx, EMB_K_ATOMIC, st);
  hipError_t e = launch_atomic_reduce(ctx->g, offsets, itype, N, B, pool, dY, inverse, num_unique, reduced_grad, st);
  if (e != hipSuccess) return hip_fail(e, "atomic reduce");
  return ok();
}

}  // extern "C"

namespace {

struct HashLayout {
  std::vector<HashMeta> meta;
  long long slots = 0;
  size_t keys_off = 0, vals_off = 0, nf_off = 0, total = 0;
};

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

// Map layout: 2^k >= 2 * rows slots per table (at least 64), keys | values |
// per-table counters. total = 0 if the slots do not fit int32.
HashLayout hash_layout(const emb_ctx* c) {
  HashLayout h;
  long long base = 0;
  for (int t = 0; t < c->g.T; ++t) {
    const long long rows = c->desc[t].rows;
    long long cap = 64;
    while (cap < 2 * rows) cap <<= 1;
    if (rows >= 0x7fffffffll || base + cap >= (1ll << 31)) return HashLayout{};
    h.meta.push_back(HashMeta{base, (uint32_t)(cap - 1), (int)rows});
    base += cap;
  }
  h.slots = base;
  h.keys_off = 0;
  h.vals_off = a256((size_t)base * 8);
  h.nf_off = a256(h.vals_off + (size_t)base * 4);
  h.total = a256(h.nf_off + (size_t)c->g.T * 4);
  return h;
}

struct HashWs {
  size_t slot_of_pos = 0, pkeys = 0, paux = 0, pval = 0, blk = 0, rank_base = 0, total = 0;
};

HashWs hash_ws(const emb_ctx* c, long long N) {
  HashWs w;
  w.slot_of_pos = 0;
  w.pkeys = a256((size_t)N * 4);
  w.paux = a256(w.pkeys + (size_t)N * 16);
  w.pval = a256(w.paux + (size_t)N * 8);
  w.blk = a256(w.pval + (size_t)N * 8);
  w.rank_base = a256(w.blk + (size_t)(N / 2048 + 2) * 4);
  w.total = a256(w.rank_base + (size_t)(c->g.T + 1) * 4);
  return w;
}

int check_lookup_args(emb_ctx* ctx, const void* ids, const void* offsets, int32_t itype, int64_t N, int32_t B) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  int rc = check_itype(itype);
  if (rc) return rc;
  if (B < 0 || N < 0) return fail(EMB_E_INVAL, "negative B or N");
  if (N >= (1ll << 31)) return fail(EMB_E_INVAL, "N must be < 2^31");
  if (B == 0 && N > 0) return fail(EMB_E_INVAL, "B == 0 with N > 0");
  if (B > 0 && !offsets) return fail(EMB_E_INVAL, "offsets is NULL");
  if (N > 0 && !ids) return fail(EMB_E_INVAL, "ids is NULL");
  if (!ctx->hash_ready) return fail(EMB_E_STATE, "no hash map memory attached");
  return EMB_OK;
}

}  // namespace

extern "C" {

size_t emb_hash_bytes(const emb_ctx* ctx) {
  if (!ctx) return 0;
  return hash_layout(ctx).total;
}

int emb_hash_attach(emb_ctx* ctx, void* mem, size_t bytes, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  const HashLayout h = hash_layout(ctx);
  if (h.total == 0) return fail(EMB_E_INVAL, "tables too large for the hash maps' int32 slot indices");
  if (!mem || !aligned(mem, 256)) return fail(EMB_E_INVAL, "map memory is NULL or not 256-byte aligned");
  if (bytes < h.total) return fail(EMB_E_WORKSPACE, "map memory of %zu bytes < %zu needed", bytes, h.total);
  int rc;
  if ((rc = ensure_device(ctx))) return rc;
  hipError_t e;
  const size_t mbytes = sizeof(HashMeta) * h.meta.size();
  if (!ctx->dev_hmeta) {
    if ((e = hipMalloc(&ctx->dev_hmeta, mbytes)) != hipSuccess) return hip_fail(e, "hipMalloc(hash layout)");
  }
  if ((e = hipMemcpy(ctx->dev_hmeta, h.meta.data(), mbytes, hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(e, "hipMemcpy(hash layout)");
  char* m = static_cast<char*>(mem);
  HashView& v = ctx->hv;
  v.meta = static_cast<const HashMeta*>(ctx->dev_hmeta);
  v.keys = reinterpret_cast<unsigned long long*>(m + h.keys_off);
  v.vals = reinterpret_cast<int*>(m + h.vals_off);
  v.next_free = reinterpret_cast<int*>(m + h.nf_off);
  v.slots = h.slots;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  KScope ks(ctx, EMB_K_HASH, st);
  if ((e = launch_hash_clear(v, ctx->g.T, st)) != hipSuccess) return hip_fail(e, "hash map reset");
  ctx->hash_ready = true;
  return ok();
}

size_t emb_hash_workspace_bytes(const emb_ctx* ctx, int64_t N) {
  if (!ctx || N < 0 || N >= (1ll << 31)) return 0;
  return hash_ws(ctx, N).total;
}

int emb_hash_translate(emb_ctx* ctx, const int64_t* ids, const void* offsets, int32_t itype, int64_t N, int32_t B,
                       int32_t insert, void* ws, size_t ws_bytes, void* rows_out, void* hip_stream) {
  int rc = check_lookup_args(ctx, ids, offsets, itype, N, B);
  if (rc) return rc;
  if (N > 0 && !rows_out) return fail(EMB_E_INVAL, "rows_out is NULL");
  const HashWs L = hash_ws(ctx, N);
  if (N > 0 && (!ws || !aligned(ws, 256))) return fail(EMB_E_INVAL, "ws is NULL or not 256-byte aligned");
  if (N > 0 && ws_bytes < L.total) return fail(EMB_E_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* w = static_cast<char*>(ws);
  KScope ks(ctx, EMB_K_HASH, st);
  HashScratch hs;
  hs.slot_of_pos = reinterpret_cast<int*>(w + L.slot_of_pos);
  hs.pkeys = reinterpret_cast<unsigned long long*>(w + L.pkeys);
  hs.paux = reinterpret_cast<int*>(w + L.paux);
  hs.pval = reinterpret_cast<int*>(w + L.pval);
  hs.blk = reinterpret_cast<uint32_t*>(w + L.blk);
  hs.rank_base = reinterpret_cast<int*>(w + L.rank_base);
  hipError_t e = launch_hash_translate(ctx->hv, ctx->dc, ctx->g.T, reinterpret_cast<const long long*>(ids), offsets,
                                       itype, (int)N, B, insert != 0, hs, rows_out, st);
  if (e != hipSuccess) return hip_fail(e, "hash translation");
  return ok();
}

int emb_hash_translate_noalloc(emb_ctx* ctx, const int64_t* ids, const void* offsets, int32_t itype, int64_t N,
                               int32_t B, int32_t insert, void* rows_out, void* hip_stream) {
  int rc = check_lookup_args(ctx, ids, offsets, itype, N, B);
  if (rc) return rc;
  if (N > 0 && !rows_out) return fail(EMB_E_INVAL, "rows_out is NULL");
  const HashWs L = hash_ws(ctx, N);
  if (L.total > kHashNoAllocBytes)
    return fail(EMB_E_WORKSPACE, "%lld lookups need %zu bytes of scratch, more than the %zu the translation "
                "without allocation holds (use emb_hash_translate with a workspace)",
                (long long)N, L.total, kHashNoAllocBytes);
  if (N == 0) return ok();
  // the maps are attached, so the context's device block exists: nothing is
  // allocated here, and the device must be the context's
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != ctx->device)
    return fail(EMB_E_INVAL, "the context lives on device %d but device %d is current", ctx->device, dev);
  void* scr = nullptr;
  if ((e = hash_noalloc_scratch(dev, &scr)) != hipSuccess) return hip_fail(e, "translation scratch address");
  char* w = static_cast<char*>(scr);
  HashScratch hs;
  hs.slot_of_pos = reinterpret_cast<int*>(w + L.slot_of_pos);
  hs.pkeys = reinterpret_cast<unsigned long long*>(w + L.pkeys);
  hs.paux = reinterpret_cast<int*>(w + L.paux);
  hs.pval = reinterpret_cast<int*>(w + L.pval);
  hs.blk = reinterpret_cast<uint32_t*>(w + L.blk);
  hs.rank_base = reinterpret_cast<int*>(w + L.rank_base);
  e = launch_hash_translate(ctx->hv, ctx->dc, ctx->g.T, reinterpret_cast<const long long*>(ids), offsets, itype,
                            (int)N, B, insert != 0, hs, rows_out, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "hash translation");
  return ok();
}

int emb_forward_pooled_hashed(emb_ctx* ctx, const int64_t* ids, const void* offsets, int32_t itype, int64_t N,
                              int32_t B, int32_t pool, float* out, void* hip_stream) {
  int rc = check_lookup_args(ctx, ids, offsets, itype, N, B);
  if (rc) return rc;
  if ((rc = check_pool(pool))) return rc;
  if (B == 0) return ok();
  if (!out || !aligned(out, 16)) return fail(EMB_E_INVAL, "out is NULL or not 16-byte aligned");
  if ((rc = ensure_device(ctx))) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  KScope ks(ctx, EMB_K_FORWARD, st);
  hipError_t e = launch_forward(ctx->g, ctx->dc, ids, offsets, itype, N, B, pool, out, 0, st,
                                nullptr, 0, &ctx->hv);
  if (e != hipSuccess) return hip_fail(e, "hashed forward");
  return ok();
}

int emb_hash_rows_used(emb_ctx* ctx, int32_t* used, void* hip_stream) {
  if (!ctx || !used) return fail(EMB_E_INVAL, "NULL argument");
  if (!ctx->hash_ready) return fail(EMB_E_STATE, "no hash map memory attached");
  hipError_t e = hipMemcpyAsync(used, ctx->hv.next_free, sizeof(int32_t) * ctx->g.T, hipMemcpyDeviceToDevice,
                                static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(rows used)");
  return ok();
}

int emb_set_shard_map(emb_ctx* ctx, const emb_shard_rule* rules, int32_t num_shards) {
  if (!ctx || !rules) return fail(EMB_E_INVAL, "NULL argument");
  if (num_shards < 1 || num_shards > EMB_MAX_SHARDS)
    return fail(EMB_E_INVAL, "num_shards must be in 1..%d", EMB_MAX_SHARDS);
  for (int t = 0; t < ctx->g.T; ++t) {
    const emb_shard_rule& r = rules[t];
    if (r.kind == EMB_SHARD_TABLE || r.kind == EMB_SHARD_ROW_CYCLIC) {
      if (r.shard < 0 || r.shard >= num_shards) return fail(EMB_E_INVAL, "table %d: shard %d not in [0, %d)", t, r.shard, num_shards);
    } else if (r.kind == EMB_SHARD_ROW_BLOCK) {
      if (r.shard != 0) return fail(EMB_E_INVAL, "table %d: row-block rule takes shard 0", t);
    } else {
      return fail(EMB_E_INVAL, "table %d: unknown shard rule kind %d", t, r.kind);
    }
  }
  ctx->shard_rules.assign(rules, rules + ctx->g.T);
  ctx->num_shards = num_shards;
  ctx->rules_dirty = true;
  return ok();
}

int emb_pack_by_shard(emb_ctx* ctx, void* ws, const float* dY, uint32_t* send_keys, int32_t* send_offsets,
                      int32_t* slot_of_unique, float* send_grad, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  if (ctx->num_shards < 1) return fail(EMB_E_STATE, "no shard map set");
  if (!ctx->last.valid || ws != ctx->last.ws)
    return fail(EMB_E_STATE, "ws is not the workspace of this context's last backward");
  if ((dY == nullptr) != (send_grad == nullptr)) return fail(EMB_E_INVAL, "dY and send_grad are given together");
  const long long N = ctx->last.N;
  if (!send_offsets) return fail(EMB_E_INVAL, "send_offsets is NULL");
  if (N > 0 && (!send_keys || !slot_of_unique)) return fail(EMB_E_INVAL, "send_keys/slot_of_unique is NULL");
  if (dY && (!aligned(dY, 16) || !aligned(send_grad, 16)))
    return fail(EMB_E_INVAL, "dY and send_grad must be 16-byte aligned");
  int rc;
  if ((rc = ensure_device(ctx))) return rc;
  hipError_t e;
  if (ctx->rules_dirty) {
    const size_t bytes = sizeof(emb_shard_rule) * ctx->shard_rules.size();
    if (!ctx->dev_rules) {
      if ((e = hipMalloc(&ctx->dev_rules, bytes)) != hipSuccess) return hip_fail(e, "hipMalloc(shard map)");
    }
    if ((e = hipMemcpy(ctx->dev_rules, ctx->shard_rules.data(), bytes, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(shard map)");
    ctx->rules_dirty = false;
  }
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int S = ctx->num_shards;
  const WsLayout L = ws_layout(ctx->g, N, ctx->last.B);
  char* w = static_cast<char*>(ws);
  uint64_t* a = reinterpret_cast<uint64_t*>(w + L.keys_a);
  uint64_t* b = reinterpret_cast<uint64_t*>(w + L.keys_b);
  if (N > 0) {
    {
      KScope ks(ctx, EMB_K_PACK, st);
      if ((e = launch_pack_dest(ctx->g, ctx->dc, static_cast<const int2*>(ctx->dev_rules), S, (int)N,
                                ctx->last.unique_keys, ctx->last.num_unique, a, st)) != hipSuccess)
        return hip_fail(e, "pack destinations");
    }
    // destinations 0..S (S = sent nowhere), sorted stably
    int bits = 1;
    while ((1 << bits) <= S) ++bits;
    const SortPlan sp = sort_plan_global(bits, N);
    const SortBufs sb{reinterpret_cast<uint32_t*>(w + L.ghist), reinterpret_cast<uint32_t*>(w + L.segbase),
                      nullptr, ctx->dc.row_off, L.ghist_cap, L.segbase_cap};
    if (int rc = run_sort(ctx, sp, sb, &a, &b, (int)N, st)) return rc;
    {
      KScope ks(ctx, EMB_K_PACK, st);
      if ((e = launch_pack_place(a, ctx->last.unique_keys, ctx->last.num_unique, (int)N, S, send_keys,
                                 slot_of_unique, st)) != hipSuccess)
        return hip_fail(e, "pack placement");
    }
  }
  {
    KScope ks(ctx, EMB_K_PACK, st);
    if ((e = launch_pack_offsets(a, (int)N, S, send_offsets, st)) != hipSuccess) return hip_fail(e, "pack offsets");
  }
  if (dY && N > 0) {
    {
      KScope ks(ctx, EMB_K_REDUCE, st);
      if ((e = launch_reduce(ctx->g, ctx->dc, 0, (int)N, ctx->last.B, ctx->last.pool, dY, L, w,
                             ctx->last.unique_keys, ctx->last.num_unique, send_grad, 0.f, 0.f, st,
                             slot_of_unique)) != hipSuccess)
        return hip_fail(e, "segment reduce into send slots");
    }
    {
      KScope ks(ctx, EMB_K_COMBINE, st);
      if ((e = launch_combine(ctx->g, ctx->dc, 0, (int)N, L, w, ctx->last.unique_keys, send_grad, 0.f, 0.f, st,
                              slot_of_unique)) != hipSuccess)
        return hip_fail(e, "segment combine into send slots");
    }
  }
  return ok();
}

int emb_check_device_error(emb_ctx* ctx, void* hip_stream) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  if (!ctx->dev_block) return ok();
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int flag = 0;
  e = hipMemcpy(&flag, ctx->dc.err_flag, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(err flag)");
  if (flag) {
    const int zero = 0;
    e = hipMemcpy(ctx->dc.err_flag, &zero, sizeof(int), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(clear err flag)");
    if (flag & 1) {
      return fail(EMB_E_BOUNDS, (flag & 2) ? "a kernel saw an index outside [0, rows), and offsets that "
                                             "break the CSR contract"
                                           : "a kernel saw an index outside [0, rows)");
    }
    if (flag & 2)
      return fail(EMB_E_INVAL, "offsets break the CSR contract (offsets[0] = 0, non-decreasing, "
                               "offsets[T*B] = N)");
    return fail(EMB_E_INVAL, "id translation saw the reserved id INT64_MIN");
  }
  return ok();
}

int emb_set_kernel_timing(emb_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(EMB_E_INVAL, "ctx is NULL");
  ctx->timing = enable != 0;
  return ok();
}

int32_t emb_probe_blocks(void) { return emb::probe_blocks(); }

int emb_probe_reads(const void* buf, int64_t nrows, int64_t stride, int32_t xcd_local, int32_t reads,
                    int32_t row_bytes, float* sink, void* hip_stream) {
  if (!buf || !sink) return fail(EMB_E_INVAL, "buf/sink is NULL");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(EMB_E_INVAL, "buf must be 16-byte and sink 4-byte aligned");
  if (row_bytes != 256 && row_bytes != 512) return fail(EMB_E_INVAL, "row_bytes %d is not 256 or 512", row_bytes);
  if (nrows < 8 || nrows >= (1ll << 32)) return fail(EMB_E_INVAL, "nrows %lld not in [8, 2^32)", (long long)nrows);
  if (stride < row_bytes || stride % 16 != 0 || stride >= (1ll << 32))
    return fail(EMB_E_INVAL, "stride %lld: need >= row_bytes, a multiple of 16, < 2^32", (long long)stride);
  if (reads < 4 || reads > 65536 || reads % 4 != 0) return fail(EMB_E_INVAL, "reads %d not in [4, 65536] / 4", reads);
  hipError_t e = emb::launch_probe_reads(buf, (uint32_t)nrows, (uint32_t)stride, xcd_local ? 1 : 0, reads, row_bytes,
                                         sink, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "probe kernel");
  return ok();
}

int emb_probe_update(const float* src, int64_t nsrc, float* a, float* b, int64_t nrows, int32_t items,
                     void* hip_stream) {
  if (!src || !a || !b) return fail(EMB_E_INVAL, "src/a/b is NULL");
  if (!aligned(src, 16) || !aligned(a, 16) || !aligned(b, 16)) return fail(EMB_E_INVAL, "src/a/b must be 16-byte aligned");
  if (nsrc < 1 || nsrc >= (1ll << 32)) return fail(EMB_E_INVAL, "nsrc %lld not in [1, 2^32)", (long long)nsrc);
  if (nrows < 1 || nrows >= (1ll << 32)) return fail(EMB_E_INVAL, "nrows %lld not in [1, 2^32)", (long long)nrows);
  if (items < 1) return fail(EMB_E_INVAL, "items %d < 1", items);
  hipError_t e = emb::launch_probe_update(src, (uint32_t)nsrc, a, b, (uint32_t)nrows, items,
                                          static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "update probe kernel");
  return ok();
}

int emb_kernel_times(emb_ctx* ctx, double* ms, int64_t* launches) {
  if (!ctx || !ms || !launches) return fail(EMB_E_INVAL, "NULL argument");
  for (int k = 0; k < EMB_K_COUNT; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  for (auto& p : ctx->pending) {
    hipError_t e = hipEventSynchronize(p.e1);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float t = 0.f;
    e = hipEventElapsedTime(&t, p.e0, p.e1);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    ms[p.kid] += t;
    launches[p.kid] += 1;
    ctx->free_events.push_back(p.e0);
    ctx->free_events.push_back(p.e1);
  }
  ctx->pending.clear();
  return ok();
}

}  // extern "C"
