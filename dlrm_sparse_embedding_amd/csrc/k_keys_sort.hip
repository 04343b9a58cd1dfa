// Backward, first half: global keys and a stable device LSD radix sort of
// (key, position) pairs.
//
// The dedup is EMBark's unique-based / reduction-based compression (RecSys'24
// article, section on embedding clusters) applied to one GPU's share: before
// any gradient is reduced or a row is written, the step's lookups are grouped
// by global key g = row_offset[t] + idx. Here the grouping is a sort: each
// lookup i becomes the 64-bit word (g << 32 | i), and an LSD radix sort over
// the low key_bits bits of g orders the words by key, with
// positions ascending inside a key because every pass is stable.
//
// Digits are 8 bits, or 9 when that saves a pass (27-bit keys: 3 passes, not 4).
// Sort pass = three kernels:
//   hist    per 2048-item tile, count digits in LDS -> ghist[digit][tile]
//   scan    one block per digit: exclusive scan of its row over tiles
//   scatter per tile: rank every item among equal digits (wave ballots give
//           the lanes holding the same digit; per-wave LDS counters carry the
//           rank across the tile's items in order), stage the tile in LDS in
//           digit order, then write runs of equal digits contiguously.
// The tile is striped per wave (item k of lane l of wave w sits at
// w*512 + k*64 + l), which is the order the ranking visits, so ranks are
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
  int32_t* bag_of_pos;
  float* inv_len;  // null unless mean pooling
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
  }
  const int lo = g0 == 0 ? 0 : __shfl(s, 0);
  const int hi = g0 + 64 < nbags ? __shfl(nxt, 63) : N;
  for (int p0 = lo; p0 < hi; p0 += 64) {  // trip count uniform: every lane joins the cross-lane reads
    const int p = p0 + lane;
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
        const long long r = ld_idx<IDX>(a.indices, p);
        if (r >= 0 && r < (long long)rowsj)
          key = roj + (uint32_t)r;
        else
          flag |= 1;
      }
      // non-temporal: the dedup's streams should not evict the rows of the
      // forward / update that may run beside it on another stream
      __builtin_nontemporal_store(((uint64_t)key << 32) | (uint32_t)p, a.keys + p);
      __builtin_nontemporal_store((int32_t)(g0 + j), a.bag_of_pos + p);
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
  a.bag_of_pos = reinterpret_cast<int32_t*>(ws + L.bag_of_pos);
  a.inv_len = pool == EMB_POOL_MEAN ? reinterpret_cast<float*>(ws + L.inv_len) : nullptr;
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

template <int RB>
__device__ __forceinline__ uint32_t digit_of(uint64_t x, int shift) {
  return (uint32_t)(x >> (32 + shift)) & ((1u << RB) - 1u);
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

template <int RB>
__global__ __launch_bounds__(256) void k_sort_hist(const uint64_t* __restrict__ keys, int N,
                                                   int shift, uint32_t* __restrict__ ghist,
                                                   int nblk) {
  constexpr int R = 1 << RB;
  __shared__ uint32_t h[R];
  for (int d = threadIdx.x; d < R; d += 256) h[d] = 0;
  __syncthreads();
  const long long base = (long long)blockIdx.x * kSortTile;
  // equal digits of a wave are counted by one LDS add from their first lane:
  // skewed keys put many lanes on one bin, which would serialise per-lane adds
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 256 + threadIdx.x;
    const bool valid = i < N;
    const uint32_t d = valid ? digit_of<RB>(keys[i], shift) : 0u;
    const uint64_t peers = digit_peers<RB>(d, valid);
    if (valid && (peers & lt) == 0) atomicAdd(&h[d], (uint32_t)__popcll(peers));
  }
  __syncthreads();
  for (int d = threadIdx.x; d < R; d += 256) ghist[(size_t)d * nblk + blockIdx.x] = h[d];
}

__global__ __launch_bounds__(256) void k_sort_scan(uint32_t* __restrict__ ghist, int nblk,
                                                   uint32_t* __restrict__ digit_tot) {
  __shared__ uint32_t lds[8];
  uint32_t* row = ghist + (size_t)blockIdx.x * nblk;
  uint32_t running = 0;
  for (int base = 0; base < nblk; base += 256 * 4) {
    uint32_t v[4];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + threadIdx.x * 4 + j;
      v[j] = i < nblk ? row[i] : 0u;
      sum += v[j];
    }
    uint32_t tot;
    uint32_t run = running + block_excl_scan_256(sum, lds, &tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + threadIdx.x * 4 + j;
      if (i < nblk) row[i] = run;
      run += v[j];
    }
    running += tot;
  }
  if (threadIdx.x == 0) digit_tot[blockIdx.x] = running;
}

template <int RB>
__global__ __launch_bounds__(256) void k_sort_scatter(const uint64_t* __restrict__ in,
                                                      uint64_t* __restrict__ out, int N, int shift,
                                                      const uint32_t* __restrict__ ghist,
                                                      const uint32_t* __restrict__ digit_tot,
                                                      int nblk) {
  constexpr int R = 1 << RB;
  constexpr int PER = R / 256;
  __shared__ uint32_t s_gbase[R];    // global start of this tile's digit-d run
  __shared__ uint32_t s_wcnt[4][R];  // per-wave digit counters, then per-wave offsets
  __shared__ uint32_t s_bexcl[R];    // tile-local start of digit d
  __shared__ uint64_t s_stage[kSortTile];
  __shared__ uint32_t s_scan[8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int blk = blockIdx.x;

  {
    uint32_t in_[PER], pre[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) in_[j] = digit_tot[tid * PER + j];
    block_excl_scan_digits<PER>(in_, pre, s_scan);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = tid * PER + j;
      s_gbase[d] = pre[j] + ghist[(size_t)d * nblk + blk];
    }
  }
#pragma unroll
  for (int w = 0; w < 4; ++w)
    for (int d = tid; d < R; d += 256) s_wcnt[w][d] = 0;
  __syncthreads();

  const long long base = (long long)blk * kSortTile + wave * (64 * kSortIPT);
  uint64_t item[kSortIPT];
  uint32_t rank[kSortIPT];
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 64 + lane;
    item[k] = i < N ? in[i] : 0ull;
  }
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const bool valid = base + k * 64 + lane < N;
    const uint32_t d = digit_of<RB>(item[k], shift);
    const uint64_t peers = digit_peers<RB>(d, valid);
    const uint32_t before = (uint32_t)__popcll(peers & lt);
    uint32_t basev = 0;
    if (valid) basev = s_wcnt[wave][d];
    rank[k] = basev + before;
    // every lane has read the counter (LDS ops of one wave complete in
    // order); the group's first lane now advances it
    __builtin_amdgcn_wave_barrier();
    if (valid && before == 0) s_wcnt[wave][d] = basev + (uint32_t)__popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  {
    uint32_t tot_[PER], pre[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = tid * PER + j;
      const uint32_t c0 = s_wcnt[0][d], c1 = s_wcnt[1][d], c2 = s_wcnt[2][d], c3 = s_wcnt[3][d];
      s_wcnt[0][d] = 0;
      s_wcnt[1][d] = c0;
      s_wcnt[2][d] = c0 + c1;
      s_wcnt[3][d] = c0 + c1 + c2;
      tot_[j] = c0 + c1 + c2 + c3;
    }
    block_excl_scan_digits<PER>(tot_, pre, s_scan);
#pragma unroll
    for (int j = 0; j < PER; ++j) s_bexcl[tid * PER + j] = pre[j];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const bool valid = base + k * 64 + lane < N;
    if (valid) {
      const uint32_t d = digit_of<RB>(item[k], shift);
      s_stage[s_bexcl[d] + s_wcnt[wave][d] + rank[k]] = item[k];
    }
  }
  __syncthreads();
  const long long rem = (long long)N - (long long)blk * kSortTile;
  const int cnt = rem < kSortTile ? (int)rem : kSortTile;
  for (int j = tid; j < cnt; j += 256) {
    const uint64_t x = s_stage[j];
    const uint32_t d = digit_of<RB>(x, shift);
    const size_t dst = (size_t)s_gbase[d] + (uint32_t)(j - (int)s_bexcl[d]);
    if (dst < (size_t)N) __builtin_nontemporal_store(x, out + dst);  // see k_keys
  }
}

int radix_bits_for(int key_bits) {
  const int p8 = (key_bits + 7) / 8;
  const int p9 = (key_bits + 8) / 9;
  return p9 < p8 ? 9 : 8;
}

hipError_t launch_sort_hist(int rb, const uint64_t* keys, int N, int shift, uint32_t* ghist,
                            int nblk, hipStream_t st) {
  if (rb == 9)
    hipLaunchKernelGGL(k_sort_hist<9>, dim3(nblk), dim3(256), 0, st, keys, N, shift, ghist, nblk);
  else
    hipLaunchKernelGGL(k_sort_hist<8>, dim3(nblk), dim3(256), 0, st, keys, N, shift, ghist, nblk);
  return hipGetLastError();
}

hipError_t launch_sort_scan(int rb, uint32_t* ghist, int nblk, uint32_t* digit_tot, hipStream_t st) {
  hipLaunchKernelGGL(k_sort_scan, dim3(1 << rb), dim3(256), 0, st, ghist, nblk, digit_tot);
  return hipGetLastError();
}

hipError_t launch_sort_scatter(int rb, const uint64_t* in, uint64_t* out, int N, int shift,
                               const uint32_t* ghist, const uint32_t* digit_tot, int nblk,
                               hipStream_t st) {
  if (rb == 9)
    hipLaunchKernelGGL(k_sort_scatter<9>, dim3(nblk), dim3(256), 0, st, in, out, N, shift, ghist,
                       digit_tot, nblk);
  else
    hipLaunchKernelGGL(k_sort_scatter<8>, dim3(nblk), dim3(256), 0, st, in, out, N, shift, ghist,
                       digit_tot, nblk);
  return hipGetLastError();
}

}  // namespace emb
