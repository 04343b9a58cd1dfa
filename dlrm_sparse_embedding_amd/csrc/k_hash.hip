// Hash-keyed lookup: 64-bit feature ids -> table rows, in front of the pooled
// forward and the backward ("Merlin HugeCTR" GTC 2022 deck, slide "HUGECTR
// EMBEDDING LAYER": a GPU hash table lookup fused with the reduction and
// concatenation; the dynamic embedding of the Sparse Operation Kit 2.0
// article: ids are not known ahead and get rows as they arrive).
//
// One open-addressing map per table in caller memory: 2^k slots (at least
// twice the table's rows), a 64-bit key per slot (kEmpty = free) and the
// int32 row of the id. Only ids that hold a row are ever stored, so a map is
// at most half full. Linear probing from a SplitMix64-mixed hash; an id
// claims a free slot with a 64-bit compare-and-swap.
//
// Rows are handed out deterministically although slots are not: per table,
// the ids first seen in this step are ranked by their first position in the
// CSR, and the id of rank k gets row next_free + k while rows last (no row
// after that). The step's new ids are gathered first in a pending map in the
// workspace, one region of twice the table's lookups per table (so it never
// fills), whose slots carry the id's first position (atomicMin) and its row.
// Steps of a translation with insertion:
//   clear   the pending map
//   probe   thread per lookup: a known id's row is final; a new id claims
//           (or finds) its pending slot and records its position
//   count   per 2048-lookup tile: lookups that are the first sight of their id
//   scan    exclusive scan of the tile counts (one block)
//   base    per table: the number of first sights before its first lookup
//   assign  per tile: rank of each first sight -> row; ids with a row are
//           inserted into the table's map
//   fill    thread per lookup: rows_out from the pending slot of a new id
//   advance per table: next_free += its first sights (capped at rows)
#include <mutex>

#include "emb_device.h"

namespace emb {

// Scratch of emb_hash_translate_noalloc, for callers that cannot allocate
// device memory: one copy per GPU, held until the process ends. Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); it takes the device address from hash_noalloc_scratch.
static __device__ __align__(256) unsigned char scratch[kHashNoAllocBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t hash_noalloc_scratch(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

constexpr int kTile = 2048;  // lookups per count / assign block (8 per thread)

// Table of lookup p: the last t < T with table_start[t] <= p.
__device__ __forceinline__ int table_of_pos(const int* s_ts, int T, int p) {
  int lo = 0, hi = T;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_ts[mid] <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <typename IDX>
__device__ __forceinline__ void stage_table_starts(const void* offsets, int T, int B, int N, int* s_ts) {
  for (int t = threadIdx.x; t <= T; t += blockDim.x)
    s_ts[t] = (int)min(max(ld_idx<IDX>(offsets, (long long)t * B), 0ll), (long long)N);
  __syncthreads();
}

struct HashArgs {
  const long long* ids;
  const void* offsets;
  const HashMeta* meta;
  unsigned long long* keys;
  int* vals;
  int* next_free;
  int* slot_of_pos;          // [N] pending slot of a new id's lookup, else -1
  unsigned long long* pkeys; // [2N] pending map: ids
  int* paux;                 // [2N] first position
  int* pval;                 // [2N] row (or -1)
  uint32_t* blk;             // [nblk + 1] tile counts, then their exclusive scan
  int* rank_base;            // [T + 1]
  void* rows_out;
  int* err;
  int N, T, B, nblk;
  int insert;
};

template <typename IDX>
__device__ __forceinline__ void store_row(void* rows_out, int p, int r) {
  reinterpret_cast<IDX*>(rows_out)[p] = (IDX)r;
}

// Finds or claims id in the pending region [base, base + cap): linear probing
// from a multiply-shift reduction of the mixed hash. -1 if the region is
// empty or full (only with offsets that break the CSR contract).
__device__ __forceinline__ long long pending_slot(unsigned long long* pkeys, long long base, long long cap,
                                                  long long id) {
  if (cap <= 0) return -1;
  long long i = (long long)(((uint64_t)(uint32_t)mix64((uint64_t)id) * (uint64_t)cap) >> 32);
  for (long long step = 0; step < cap; ++step) {
    const long long slot = base + i;
    const long long k = (long long)__hip_atomic_load(pkeys + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k == id) return slot;
    if (k == kEmpty) {
      const unsigned long long old = atomicCAS(pkeys + slot, (unsigned long long)kEmpty, (unsigned long long)id);
      if ((long long)old == kEmpty || (long long)old == id) return slot;
    }
    i = i + 1 == cap ? 0 : i + 1;
  }
  return -1;
}

__global__ __launch_bounds__(256) void k_pend_clear(unsigned long long* pkeys, int* paux, long long n) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    pkeys[i] = (unsigned long long)kEmpty;
    paux[i] = 0x7fffffff;
  }
}

template <typename IDX>
__global__ __launch_bounds__(256) void k_hash_probe(HashArgs a) {
  extern __shared__ int s_ts[];
  stage_table_starts<IDX>(a.offsets, a.T, a.B, a.N, s_ts);
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.N) return;
  const int t = table_of_pos(s_ts, a.T, p);
  const long long id = a.ids[p];
  int row = -1, sop = -1, flag = 0;
  if (id == kEmpty) {
    flag = 4;  // the reserved free-slot key is not a valid id
  } else {
    const long long slot = find_slot(a.meta[t], a.keys, id, false);
    if (slot >= 0) {
      row = a.vals[slot];
    } else if (a.insert) {
      const long long lo = s_ts[t], hi = s_ts[t + 1];
      const long long ps = pending_slot(a.pkeys, 2 * lo, 2 * (hi - lo), id);
      if (ps >= 0) {
        atomicMin(a.paux + ps, p);
        sop = (int)ps;
      }
    }
  }
  a.slot_of_pos[p] = sop;
  store_row<IDX>(a.rows_out, p, row);
  if (flag) atomicOr(a.err, flag);
}

__device__ __forceinline__ bool first_sight(const HashArgs& a, int p) {
  const int s = a.slot_of_pos[p];
  return s >= 0 && a.paux[s] == p;
}

__global__ __launch_bounds__(256) void k_hash_count(HashArgs a) {
  __shared__ uint32_t lds[8];
  const int p0 = blockIdx.x * kTile + threadIdx.x * 8;
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (p0 + k < a.N) c += first_sight(a, p0 + k);
  uint32_t tot;
  block_excl_scan_256(c, lds, &tot);
  if (threadIdx.x == 0) a.blk[blockIdx.x] = tot;
}

// One block: exclusive scan of the nblk tile counts in place; blk[nblk] = total.
__global__ __launch_bounds__(256) void k_hash_scan(HashArgs a) {
  __shared__ uint32_t lds[8];
  const int per = (a.nblk + 255) / 256;
  const int b0 = threadIdx.x * per;
  uint32_t s = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < a.nblk) s += a.blk[b0 + i];
  uint32_t tot;
  uint32_t run = block_excl_scan_256(s, lds, &tot);
  for (int i = 0; i < per; ++i) {
    if (b0 + i < a.nblk) {
      const uint32_t v = a.blk[b0 + i];
      a.blk[b0 + i] = run;
      run += v;
    }
  }
  if (threadIdx.x == 0) a.blk[a.nblk] = tot;
}

// Block t (0..T): first sights before the table's first lookup.
template <typename IDX>
__global__ __launch_bounds__(256) void k_hash_base(HashArgs a) {
  __shared__ uint32_t lds[8];
  const int t = blockIdx.x;
  const int start = t == a.T ? a.N : (int)min(max(ld_idx<IDX>(a.offsets, (long long)t * a.B), 0ll), (long long)a.N);
  const int b = start / kTile;
  uint32_t c = 0;
  for (int p = b * kTile + threadIdx.x; p < start; p += 256) c += first_sight(a, p);
  uint32_t tot;
  block_excl_scan_256(c, lds, &tot);
  if (threadIdx.x == 0) a.rank_base[t] = (int)(a.blk[min(b, a.nblk)] + tot);
}

template <typename IDX>
__global__ __launch_bounds__(256) void k_hash_assign(HashArgs a) {
  extern __shared__ int s_ts[];
  __shared__ uint32_t lds[8];
  stage_table_starts<IDX>(a.offsets, a.T, a.B, a.N, s_ts);
  const int p0 = blockIdx.x * kTile + threadIdx.x * 8;
  bool f[8];
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f[k] = p0 + k < a.N && first_sight(a, p0 + k);
    c += f[k];
  }
  uint32_t tot;
  uint32_t rank = a.blk[blockIdx.x] + block_excl_scan_256(c, lds, &tot);
  int flag = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (f[k]) {
      const int p = p0 + k;
      const int t = table_of_pos(s_ts, a.T, p);
      const long long r = (long long)a.next_free[t] + ((long long)rank - a.rank_base[t]);
      int row = -1;
      if (r < a.meta[t].rows) {
        // first sights are distinct ids of the table: each is inserted once,
        // and the map (2x rows slots, at most rows ids) always has room
        const long long slot = find_slot(a.meta[t], a.keys, a.ids[p], true);
        if (slot >= 0) {
          a.vals[slot] = (int)r;
          row = (int)r;
        } else {
          flag = 4;
        }
      }
      a.pval[a.slot_of_pos[p]] = row;
      ++rank;
    }
  }
  if (flag) atomicOr(a.err, flag);
}

template <typename IDX>
__global__ __launch_bounds__(256) void k_hash_fill(HashArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.N) return;
  const int s = a.slot_of_pos[p];
  if (s < 0) return;
  store_row<IDX>(a.rows_out, p, a.pval[s]);
}

__global__ __launch_bounds__(256) void k_hash_advance(HashArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  const long long n = (long long)a.next_free[t] + (a.rank_base[t + 1] - a.rank_base[t]);
  a.next_free[t] = (int)min(n, (long long)a.meta[t].rows);
}

// Map reset: every slot free, next_free = 0.
__global__ __launch_bounds__(256) void k_hash_clear(unsigned long long* keys, int* vals, long long slots,
                                                    int* next_free, int T) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < slots; i += stride) {
    keys[i] = (unsigned long long)kEmpty;
    vals[i] = -1;
  }
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < T; t += stride) next_free[t] = 0;
}

// ---------------------------------------------------------------------------

static int grid_for(long long n) {
  const long long want = (n + 255) / 256;
  return (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
}

hipError_t launch_hash_clear(const HashView& h, int T, hipStream_t st) {
  hipLaunchKernelGGL(k_hash_clear, dim3(grid_for(h.slots)), dim3(256), 0, st, h.keys, h.vals, h.slots, h.next_free, T);
  return hipGetLastError();
}

hipError_t launch_hash_translate(const HashView& h, const DevCtx& dc, int T, const long long* ids,
                                 const void* offsets, int itype, int N, int B, bool insert, const HashScratch& w,
                                 void* rows_out, hipStream_t st) {
  HashArgs a;
  a.ids = ids;
  a.offsets = offsets;
  a.meta = h.meta;
  a.keys = h.keys;
  a.vals = h.vals;
  a.next_free = h.next_free;
  a.slot_of_pos = w.slot_of_pos;
  a.pkeys = w.pkeys;
  a.paux = w.paux;
  a.pval = w.pval;
  a.blk = w.blk;
  a.rank_base = w.rank_base;
  a.rows_out = rows_out;
  a.err = dc.err_flag;
  a.N = N;
  a.T = T;
  a.B = B;
  a.nblk = (N + kTile - 1) / kTile;
  a.insert = insert ? 1 : 0;
  if (N == 0) return hipSuccess;
  const size_t smem = (size_t)(T + 1) * 4;
  const int g1 = (N + 255) / 256;
  if (insert)
    hipLaunchKernelGGL(k_pend_clear, dim3(grid_for(2ll * N)), dim3(256), 0, st, w.pkeys, w.paux, 2ll * N);
#define HT(IDX)                                                                                        \
  hipLaunchKernelGGL(k_hash_probe<IDX>, dim3(g1), dim3(256), smem, st, a);                            \
  if (insert) {                                                                                        \
    hipLaunchKernelGGL(k_hash_count, dim3(a.nblk), dim3(256), 0, st, a);                              \
    hipLaunchKernelGGL(k_hash_scan, dim3(1), dim3(256), 0, st, a);                                    \
    hipLaunchKernelGGL(k_hash_base<IDX>, dim3(T + 1), dim3(256), 0, st, a);                           \
    hipLaunchKernelGGL(k_hash_assign<IDX>, dim3(a.nblk), dim3(256), smem, st, a);                     \
    hipLaunchKernelGGL(k_hash_fill<IDX>, dim3(g1), dim3(256), 0, st, a);                              \
    hipLaunchKernelGGL(k_hash_advance, dim3((T + 255) / 256), dim3(256), 0, st, a);                   \
  }
  if (itype == EMB_I32) {
    HT(int32_t)
  } else {
    HT(int64_t)
  }
#undef HT
  return hipGetLastError();
}

}  // namespace emb
