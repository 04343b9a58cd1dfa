// Backward, first half: global keys and a stable device LSD radix sort of
// (key, bag) pairs.
//
// The dedup is EMBark's unique-based / reduction-based compression (RecSys'24
// article, section on embedding clusters) applied to one GPU's share: before
// any gradient is reduced or a row is written, the step's lookups are grouped
// by global key g = row_offset[t] + idx. Here the grouping is a sort: lookup
// i of bag b becomes the 64-bit word (g << 32 | b), and an LSD radix sort
// orders the words by key, with positions (and so bags) ascending inside a
// key because every pass is stable.
//
// The sort runs over segments of positions, each sorted on its own:
//   global     one segment [0, N), digits of the key itself (key_bits bits);
//   by table   the lookups are table-major, so table t's positions already
//              form one contiguous segment and every key in it lies in
//              [row_offset[t], row_offset[t+1]): sorting each segment on the
//              row bits (key - row_offset[t]) gives the same order as the
//              global sort with fewer bits (100 tables of 1M rows: 20 bits
//              in 2 passes instead of 27 bits in 3).
// Digits are 8 to 10 bits, as few passes as 10-bit digits allow (wider
// digits cost more per pass than the pass they save: more counters per tile
// to write and scan, shorter runs to scatter).
// Tiles hold 2048 items (8 per thread), or 4096 for sorts of 16 Mi items and
// more (longer runs per digit, half the counters; below that, fewer blocks
// would hide less latency).
// Sort pass = three kernels:
//   hist    per tile, count digits in LDS -> ghist[digit][tile]
//           (tiles never straddle segments; consecutive tiles run on one
//           XCD, so their counts share cache lines in one L2, and so do the
//           runs that neighbouring tiles scatter to one digit's range)
//   scan    one block per digit: exclusive scan of its row over tiles, plus
//           the value at each segment's first tile (segbase)
//   scatter per tile: rank every item among equal digits (wave ballots give
//           the lanes holding the same digit; per-wave LDS counters carry the
//           rank across the tile's items in order), stage the tile in LDS in
//           digit order, then write runs of equal digits contiguously to
//           segment start + digits below + this digit's tiles before.
// The tile is striped per wave (item k of lane l of wave w sits at
// w*64*IPT + k*64 + l), which is the order the ranking visits, so ranks are
// stable.
#include "emb_device.h"

namespace emb {

// ---------------------------------------------------------------------------
// keys
// ---------------------------------------------------------------------------

struct KeysArgs {
  const void* indices;
  const void* offsets;
  const uint32_t* row_off;
  uint64_t* keys;
  uint32_t* key_of_pos;
  float* inv_len;  // null unless mean pooling
  int32_t* seg_start;  // [T] first position of each table's bags (clamped offsets[t*B])
  int32_t* unit_grp;   // [groups] 1 if every bag of the group is [b, b+1) (its one lookup is position b)
  int* err;
  long long N;
  int T, B;
  uint32_t total_rows;
};

// One wave per group of 64 consecutive bags (table-major bag ids g0 ..
// g0+63). Lane j holds bag g0+j's clamped range [s_j, e_j); the wave then
// walks the group's positions 64 at a time, so index loads and key / bag
// stores are coalesced whatever the bag lengths, and finds each position's
// bag as the last lane whose start is <= the position (a 6-step binary search
// over the lanes' starts by cross-lane reads).
//
// Group g owns positions [lo_g, hi_g) with lo_g = clamp(offsets[g0]) (0 for
// the first group) and hi_g = lo of the next group (N for the last). These
// intervals cover [0, N) for any offsets, so every position gets an in-range
// key and bag even when the offsets break the contract; such offsets raise
// bit 2 of the error flag, an index outside its table bit 1.
template <typename IDX>
__global__ __launch_bounds__(256) void k_keys(KeysArgs a) {
  const long long nbags = (long long)a.T * a.B;
  const long long g0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  if (g0 >= nbags) return;  // uniform over the wave
  const int lane = threadIdx.x & 63;
  const long long bag = g0 + lane;
  const int N = (int)a.N;
  int s = N, e = N, nxt = N, flag = 0;  // lanes past the last bag: empty at N
  uint32_t ro = 0, rows = 0;
  if (bag < nbags) {
    const int t = (int)(bag / a.B);
    const long long o0 = ld_idx<IDX>(a.offsets, bag);
    const long long o1 = ld_idx<IDX>(a.offsets, bag + 1);
    if (o0 < 0 || o1 < o0 || o1 > N || (bag == 0 && o0 != 0) || (bag == nbags - 1 && o1 != N))
      flag |= 2;
    s = (int)min(max(o0, 0ll), (long long)N);
    nxt = (int)min(max(o1, 0ll), (long long)N);
    e = max(nxt, s);
    ro = a.row_off[t];
    rows = a.row_off[t + 1] - ro;
    if (a.inv_len) a.inv_len[bag] = e > s ? __fdiv_rn(1.0f, (float)(e - s)) : 0.f;
    if (bag - (long long)t * a.B == 0) a.seg_start[t] = s;
  }
  {
    const bool unit = bag >= nbags || (s == bag && nxt == bag + 1);
    const uint64_t bu = __ballot(unit);
    if (lane == 0) a.unit_grp[g0 / 64] = bu == ~0ull ? 1 : 0;
  }
  const int lo = g0 == 0 ? 0 : __shfl(s, 0);
  const int hi = g0 + 64 < nbags ? __shfl(nxt, 63) : N;
  // Each pass reads the next pass's row indices (at clamped positions, so
  // the load needs no branch) while it finds bags and stores keys: a long
  // group waits on one index round trip, not one per 64 positions.
  long long rnext = lo < hi ? ld_idx<IDX>(a.indices, min(lo + lane, hi - 1)) : 0;
  for (int p0 = lo; p0 < hi; p0 += 64) {  // trip count uniform: every lane joins the cross-lane reads
    const int p = p0 + lane;
    const long long r = rnext;
    rnext = ld_idx<IDX>(a.indices, min(p + 64, hi - 1));
    int j = 0;
#pragma unroll
    for (int st = 32; st >= 1; st >>= 1) {
      if (__shfl(s, j + st) <= p) j += st;
    }
    const int sj = __shfl(s, j), ej = __shfl(e, j);
    const uint32_t roj = __shfl(ro, j), rowsj = __shfl(rows, j);
    if (p < hi) {
      uint32_t key = a.total_rows;  // sentinel: sorts last, never applied
      if (p < sj || p >= ej) {
        flag |= 2;
      } else {
        if (r >= 0 && r < (long long)rowsj)
          key = roj + (uint32_t)r;
        else
          flag |= 1;
      }
      // The sort word carries the bag (the sort is stable, so a key's bags
      // stay ascending); the position's key is kept in input order for the
      // inverse, a sentinel as total_rows + its table. Non-temporal: the
      // dedup's streams should not evict the rows of the forward / update
      // that may run beside it on another stream.
      const uint32_t bg = (uint32_t)(g0 + j);
      __builtin_nontemporal_store(((uint64_t)key << 32) | bg, a.keys + p);
      const uint32_t kp = key < a.total_rows ? key : a.total_rows + bg / (uint32_t)a.B;
      __builtin_nontemporal_store(kp, a.key_of_pos + p);
    }
  }
  if (flag) atomicOr(a.err, flag);
}

hipError_t launch_keys(const Geom& g, const DevCtx& dc, const void* indices, const void* offsets,
                       int itype, long long N, int B, int pool, const WsLayout& L, char* ws,
                       hipStream_t st) {
  KeysArgs a;
  a.indices = indices;
  a.offsets = offsets;
  a.row_off = dc.row_off;
  a.keys = reinterpret_cast<uint64_t*>(ws + L.keys_a);
  a.key_of_pos = reinterpret_cast<uint32_t*>(ws + L.key_of_pos);
  a.inv_len = pool == EMB_POOL_MEAN ? reinterpret_cast<float*>(ws + L.inv_len) : nullptr;
  a.seg_start = reinterpret_cast<int32_t*>(ws + L.seg_start);
  a.unit_grp = reinterpret_cast<int32_t*>(ws + L.unit_grp);
  a.err = dc.err_flag;
  a.N = N;
  a.T = g.T;
  a.B = B;
  a.total_rows = g.total_rows;
  const long long bags = (long long)g.T * B;
  const int grid = ceil_div(bags, 256);  // 4 waves x 64 bags per block
  if (grid == 0) return hipSuccess;
  if (itype == EMB_I32)
    hipLaunchKernelGGL(k_keys<int32_t>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_keys<int64_t>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// radix sort
// ---------------------------------------------------------------------------

// Segment map of one sort, rebuilt in LDS by every block of the table-
// segmented sort: segment t covers positions [sb[t], sb[t+1]) and tiles
// [tf[t], tf[t+1]). sb is the running maximum of the clamped table starts
// with sb[0] = 0 and sb[S] = N, so the segments partition [0, N) whatever the
// offsets were (with offsets that break the CSR contract, a segment may hold
// keys of another table; they take the largest row value, see local_of).
struct SegLds {
  int sb[kSegMaxTables + 1];
  int tf[kSegMaxTables + 1];
};

struct SortKArgs {
  const int32_t* seg_start;  // [S] (table-segmented) or null (one segment)
  const uint32_t* row_off;   // [S+1] (table-segmented)
  uint32_t* ghist;           // [R][nblk] per-tile digit counts, scanned in place
  uint32_t* segbase;         // [S+1][R] scanned count at each segment's first tile
  int S;                     // segments
  int nblk;                  // tiles in the grid (multiple of 8)
  int N;
  int tile;                  // items per tile: 256 x items per thread
  uint32_t vmax;             // row value of a key outside its segment's table
};

// Builds the segment map (wave 0; every thread must call: barriers inside).
__device__ void build_seg_map(const SortKArgs& a, SegLds& m) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int carry = 0;
    for (int c = 0; c <= a.S; c += 64) {
      const int t = c + lane;
      int v = a.N;
      if (t == 0) v = 0;
      else if (t < a.S) v = min(max(a.seg_start[t], 0), a.N);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(v, d, 64);
        if (lane >= d) v = max(v, y);
      }
      v = max(v, carry);
      if (t <= a.S) m.sb[t] = v;
      carry = __shfl(v, 63, 64);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    int carry = 0;
    for (int c = 0; c < a.S; c += 64) {
      const int t = c + lane;
      const int n = t < a.S ? (m.sb[t + 1] - m.sb[t] + a.tile - 1) / a.tile : 0;
      int x = n;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (t < a.S) m.tf[t] = carry + x - n;
      carry += __shfl(x, 63, 64);
    }
    if (lane == 0) m.tf[a.S] = carry;
  }
  __syncthreads();
}

// The tile a block works on: its segment and position range [lo, hi)
// (empty past the last tile).
struct TileRange {
  int seg, lo, hi;
};

__device__ __forceinline__ TileRange tile_range(const SortKArgs& a, const SegLds& m, int k) {
  TileRange r{0, a.N, a.N};
  if (a.seg_start) {
    if (k >= m.tf[a.S]) return r;
    int lo = 0, hi = a.S;  // tf[lo] <= k < tf[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (m.tf[mid] <= k) lo = mid;
      else hi = mid;
    }
    r.seg = lo;
    r.lo = m.sb[lo] + (k - m.tf[lo]) * a.tile;
    r.hi = min(r.lo + a.tile, m.sb[lo + 1]);
  } else {
    const long long s0 = (long long)k * a.tile;
    if (s0 < a.N) {
      r.lo = (int)s0;
      r.hi = (int)min(s0 + a.tile, (long long)a.N);
    }
  }
  return r;
}

// Value sorted for a word: its key (global sort), or its row within the
// segment's table [lo, lo + span) -- a key outside that range (the invalid-
// index sentinel) takes vmax, after every row of the table.
__device__ __forceinline__ uint32_t local_of(uint64_t x, uint32_t lo, uint32_t span, uint32_t vmax) {
  const uint32_t v = (uint32_t)(x >> 32) - lo;
  return v < span ? v : vmax;
}

template <int RB>
__device__ __forceinline__ uint32_t digit_of(uint32_t v, int shift) {
  return (v >> shift) & ((1u << RB) - 1u);
}

// Mask of the wave's lanes that are valid and hold the same RB-bit digit as
// this lane (one ballot per digit bit).
template <int RB>
__device__ __forceinline__ uint64_t digit_peers(uint32_t d, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bb = __ballot(bit);
    peers &= bit ? bb : ~bb;
  }
  return peers;
}

// Exclusive scan over R = 256 * PER digits held PER-per-thread (thread i owns
// digits i*PER .. i*PER+PER-1). Contains __syncthreads.
template <int PER>
__device__ __forceinline__ void block_excl_scan_digits(const uint32_t* in, uint32_t* out, uint32_t* lds) {
  uint32_t v[PER], sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    v[j] = in[j];
    sum += v[j];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan_256(sum, lds, &tot);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    out[j] = run;
    run += v[j];
  }
}

// Block of tile k: consecutive tiles on one XCD (a.nblk % 8 == 0).
__device__ __forceinline__ int sort_tile_of_block(const SortKArgs& a) {
  return xcd_remap((int)blockIdx.x, a.nblk);
}

// Row range of the block's segment (the whole key range in the global sort).
__device__ __forceinline__ void seg_rows(const SortKArgs& a, int seg, uint32_t* lo, uint32_t* span) {
  if (a.seg_start) {
    *lo = a.row_off[seg];
    *span = a.row_off[seg + 1] - *lo;
  } else {
    *lo = 0;
    *span = 0xffffffffu;
  }
}

template <int RB, int IPT>
__global__ __launch_bounds__(256) void k_sort_hist(const uint64_t* __restrict__ keys, int shift, SortKArgs a) {
  constexpr int R = 1 << RB;
  __shared__ uint32_t h[R];
  __shared__ SegLds m;
  for (int d = threadIdx.x; d < R; d += 256) h[d] = 0;
  if (a.seg_start) build_seg_map(a, m);
  const int k = sort_tile_of_block(a);
  const TileRange r = tile_range(a, m, k);
  uint32_t lo = 0, span = 0;
  if (r.lo < r.hi) seg_rows(a, r.seg, &lo, &span);
  __syncthreads();
  // All of the tile's words are loaded before any is counted: from the
  // tile's start (a scalar base) at clamped 32-bit offsets, so the loads need
  // no branch and few address registers and go out back to back (one memory
  // round trip per tile, not one per item).
  uint64_t w[IPT];
  const int t_lo = __builtin_amdgcn_readfirstlane(r.lo);
  const int t_n = __builtin_amdgcn_readfirstlane(r.hi - r.lo);
  if (t_n > 0) {
    const uint64_t* kb = keys + t_lo;
#pragma unroll
    for (int j = 0; j < IPT; ++j) w[j] = kb[min(j * 256 + (int)threadIdx.x, t_n - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < IPT; ++j) w[j] = 0;
  }
  // equal digits of a wave are counted by one LDS add from their first lane:
  // skewed keys put many lanes on one bin, which would serialise per-lane adds
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = r.lo + j * 256 + threadIdx.x;
    const bool valid = i < r.hi;
    const uint32_t d = valid ? digit_of<RB>(local_of(w[j], lo, span, a.vmax), shift) : 0u;
    const uint64_t peers = digit_peers<RB>(d, valid);
    if (valid && (peers & lt) == 0) atomicAdd(&h[d], (uint32_t)__popcll(peers));
  }
  __syncthreads();
  for (int d = threadIdx.x; d < R; d += 256) a.ghist[(size_t)d * a.nblk + k] = h[d];
}

// One block per digit.
template <int RB>
__global__ __launch_bounds__(256) void k_sort_scan(SortKArgs a) {
  constexpr int R = 1 << RB;
  __shared__ uint32_t lds[8];
  __shared__ SegLds m;
  __shared__ uint32_t s_base[kSegMaxTables + 1];
  const int d = (int)blockIdx.x;
  uint32_t* row = a.ghist + (size_t)d * a.nblk;
  if (a.seg_start) {
    build_seg_map(a, m);
  } else if (threadIdx.x == 0) {
    m.tf[0] = 0;
    m.tf[1] = a.nblk;
  }
  __syncthreads();
  // The row is scanned 1024 tiles at a time; the next window's counts are
  // loaded (at clamped indices, without a branch) while this one is scanned,
  // so a window costs a block scan, not a memory round trip. Each window's
  // exclusive prefixes are kept in LDS, where the segments whose first tile
  // falls in the window read their base.
  constexpr int W = 256 * 4;
  __shared__ uint32_t s_ex[W];
  const int last = a.nblk - 1;
  uint32_t running = 0;
  // raw loads; counts past the row's end are masked where they are used, so
  // that nothing waits on the prefetch before the next window
  uint32_t xn[4] = {0u, 0u, 0u, 0u};
  if (last >= 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) xn[j] = row[min((int)threadIdx.x * 4 + j, last)];
  }
  for (int base = 0; base < a.nblk; base += W) {
    uint32_t v[4];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = base + (int)threadIdx.x * 4 + j <= last ? xn[j] : 0u;
      sum += v[j];
    }
    if (base + W <= last) {  // uniform over the block
#pragma unroll
      for (int j = 0; j < 4; ++j) xn[j] = row[min(base + W + (int)threadIdx.x * 4 + j, last)];
    }
    uint32_t tot;
    uint32_t run = running + block_excl_scan_256(sum, lds, &tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + threadIdx.x * 4 + j;
      if (i < a.nblk) row[i] = run;
      s_ex[threadIdx.x * 4 + j] = run;
      run += v[j];
    }
    __syncthreads();
    // segments whose first tile lies in this window (several share a tile
    // when segments are empty)
    for (int t = threadIdx.x; t <= a.S; t += 256) {
      const int f = m.tf[t];
      if (f >= base && f < base + W && f < a.nblk) s_base[t] = s_ex[f - base];
    }
    __syncthreads();
    running += tot;
  }
  for (int t = threadIdx.x; t <= a.S; t += 256)
    if (m.tf[t] >= a.nblk) s_base[t] = running;
  __syncthreads();
  for (int t = threadIdx.x; t <= a.S; t += 256) a.segbase[(size_t)t * R + d] = s_base[t];
}

template <int RB, int IPT>
__global__ __launch_bounds__(256) void k_sort_scatter(const uint64_t* __restrict__ in,
                                                      uint64_t* __restrict__ out, int shift,
                                                      SortKArgs a) {
  constexpr int R = 1 << RB;
  constexpr int PER = R / 256;
  __shared__ uint32_t s_gbase[R];    // global start of this tile's digit-d run
  __shared__ uint16_t s_wcnt[4][R];  // per-wave digit counters, then per-wave offsets
  __shared__ uint16_t s_bexcl[R];    // tile-local start of digit d
  __shared__ uint64_t s_stage[256 * IPT];
  __shared__ uint32_t s_scan[8];
  __shared__ SegLds m;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (a.seg_start) build_seg_map(a, m);
  const int k = sort_tile_of_block(a);
  const TileRange r = tile_range(a, m, k);
  if (r.lo >= r.hi) return;  // uniform over the block, after the map's barriers
  uint32_t lo, span;
  seg_rows(a, r.seg, &lo, &span);
  const int sb = a.seg_start ? m.sb[r.seg] : 0;

  // The tile's words and the digit bases are all loaded before anything is
  // computed: the words from the tile's start (a scalar base) at clamped
  // 32-bit offsets, so the loads go out back to back and their latency
  // overlaps the bases' scan.
  const int base = r.lo + wave * (64 * IPT);
  uint64_t item[IPT];
  uint32_t rank[IPT];
  {
    const int t_lo = __builtin_amdgcn_readfirstlane(r.lo);
    const int t_n = __builtin_amdgcn_readfirstlane(r.hi - r.lo);
    const uint64_t* tb = in + t_lo;
#pragma unroll
    for (int j = 0; j < IPT; ++j) item[j] = tb[min(wave * (64 * IPT) + j * 64 + lane, t_n - 1)];
  }
  {
    // digit d's run of this tile starts at: segment start + items of the
    // segment with smaller digits + items of digit d in the segment's tiles
    // before this one
    const uint32_t* b0 = a.segbase + (size_t)r.seg * R;
    const uint32_t* b1 = b0 + R;
    const uint32_t* gh = a.ghist + k;
    uint32_t in_[PER], pre[PER], g_[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int dd = tid * PER + j;
      const uint32_t lo0 = b0[dd];
      in_[j] = b1[dd] - lo0;
      g_[j] = gh[(size_t)dd * a.nblk] - lo0;
    }
    block_excl_scan_digits<PER>(in_, pre, s_scan);
#pragma unroll
    for (int j = 0; j < PER; ++j) s_gbase[tid * PER + j] = (uint32_t)sb + pre[j] + g_[j];
  }
#pragma unroll
  for (int w = 0; w < 4; ++w)
    for (int dd = tid; dd < R; dd += 256) s_wcnt[w][dd] = 0;
  __syncthreads();

  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool valid = base + j * 64 + lane < r.hi;
    const uint32_t d = digit_of<RB>(local_of(item[j], lo, span, a.vmax), shift);
    const uint64_t peers = digit_peers<RB>(d, valid);
    const uint32_t before = (uint32_t)__popcll(peers & lt);
    uint32_t basev = 0;
    if (valid) basev = s_wcnt[wave][d];
    rank[j] = basev + before;
    // every lane has read the counter (LDS ops of one wave complete in
    // order); the group's first lane now advances it
    __builtin_amdgcn_wave_barrier();
    if (valid && before == 0) s_wcnt[wave][d] = (uint16_t)(basev + (uint32_t)__popcll(peers));
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  {
    uint32_t tot_[PER], pre[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int dd = tid * PER + j;
      const uint32_t c0 = s_wcnt[0][dd], c1 = s_wcnt[1][dd], c2 = s_wcnt[2][dd], c3 = s_wcnt[3][dd];
      s_wcnt[0][dd] = 0;
      s_wcnt[1][dd] = (uint16_t)c0;
      s_wcnt[2][dd] = (uint16_t)(c0 + c1);
      s_wcnt[3][dd] = (uint16_t)(c0 + c1 + c2);
      tot_[j] = c0 + c1 + c2 + c3;
    }
    block_excl_scan_digits<PER>(tot_, pre, s_scan);
#pragma unroll
    for (int j = 0; j < PER; ++j) s_bexcl[tid * PER + j] = (uint16_t)pre[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool valid = base + j * 64 + lane < r.hi;
    if (valid) {
      const uint32_t d = digit_of<RB>(local_of(item[j], lo, span, a.vmax), shift);
      s_stage[s_bexcl[d] + s_wcnt[wave][d] + rank[j]] = item[j];
    }
  }
  __syncthreads();
  const int cnt = r.hi - r.lo;
  for (int j = tid; j < cnt; j += 256) {
    const uint64_t x = s_stage[j];
    const uint32_t d = digit_of<RB>(local_of(x, lo, span, a.vmax), shift);
    const uint32_t dst = s_gbase[d] + (uint32_t)(j - (int)s_bexcl[d]);
    // ordinary stores: neighbouring tiles run on one XCD and write adjacent
    // runs of a digit, which then merge in its L2 (a non-temporal store would
    // send each short run to memory as a partial line)
    if (dst < (uint32_t)a.N) out[dst] = x;
  }
}

namespace {

SortKArgs kargs(const SortPlan& p, const SortBufs& b, int N) {
  SortKArgs a;
  a.seg_start = p.seg ? b.seg_start : nullptr;
  a.row_off = b.row_off;
  a.ghist = b.ghist;
  a.segbase = b.segbase;
  a.S = p.S;
  a.nblk = p.nblk;
  a.N = N;
  a.tile = 256 * p.ipt;
  a.vmax = p.seg ? (1u << p.bits) - 1u : 0xffffffffu;
  return a;
}

}  // namespace

#define EMB_SORT_DISPATCH(RBV, KERNEL, GRID, ...)                                    \
  switch (RBV) {                                                                     \
    case 8: hipLaunchKernelGGL(KERNEL<8>, GRID, dim3(256), 0, st, __VA_ARGS__); break;   \
    case 9: hipLaunchKernelGGL(KERNEL<9>, GRID, dim3(256), 0, st, __VA_ARGS__); break;   \
    default: hipLaunchKernelGGL(KERNEL<10>, GRID, dim3(256), 0, st, __VA_ARGS__); break; \
  }
#define EMB_SORT_DISPATCH_IPT(RBV, IPTV, KERNEL, GRID, ...)                          \
  switch (RBV * 100 + IPTV) {                                                        \
    case 808: hipLaunchKernelGGL((KERNEL<8, 8>), GRID, dim3(256), 0, st, __VA_ARGS__); break;   \
    case 908: hipLaunchKernelGGL((KERNEL<9, 8>), GRID, dim3(256), 0, st, __VA_ARGS__); break;   \
    case 1008: hipLaunchKernelGGL((KERNEL<10, 8>), GRID, dim3(256), 0, st, __VA_ARGS__); break; \
    case 816: hipLaunchKernelGGL((KERNEL<8, 16>), GRID, dim3(256), 0, st, __VA_ARGS__); break;  \
    case 916: hipLaunchKernelGGL((KERNEL<9, 16>), GRID, dim3(256), 0, st, __VA_ARGS__); break;  \
    default: hipLaunchKernelGGL((KERNEL<10, 16>), GRID, dim3(256), 0, st, __VA_ARGS__); break;  \
  }

hipError_t launch_sort_hist(const SortPlan& p, const SortBufs& b, const uint64_t* keys, int N, int shift,
                            hipStream_t st) {
  const SortKArgs a = kargs(p, b, N);
  EMB_SORT_DISPATCH_IPT(p.rb, p.ipt, k_sort_hist, dim3(p.nblk), keys, shift, a);
  return hipGetLastError();
}

hipError_t launch_sort_scan(const SortPlan& p, const SortBufs& b, int N, hipStream_t st) {
  const SortKArgs a = kargs(p, b, N);
  EMB_SORT_DISPATCH(p.rb, k_sort_scan, dim3(1u << p.rb), a);
  return hipGetLastError();
}

hipError_t launch_sort_scatter(const SortPlan& p, const SortBufs& b, const uint64_t* in, uint64_t* out, int N,
                               int shift, hipStream_t st) {
  const SortKArgs a = kargs(p, b, N);
  EMB_SORT_DISPATCH_IPT(p.rb, p.ipt, k_sort_scatter, dim3(p.nblk), in, out, shift, a);
  return hipGetLastError();
}

#undef EMB_SORT_DISPATCH
#undef EMB_SORT_DISPATCH_IPT

}  // namespace emb
