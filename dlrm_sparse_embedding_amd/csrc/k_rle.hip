// Backward, second half of the dedup: run-length encoding of the sorted
// (key, bag) words into the unique keys, their counts, each lookup's
// segment id (inverse) and the chunking of every segment used by the
// gradient reduction.
//
// The inverse: on a batch of one lookup per bag at the bag's own index
// (one-hot features) a word's bag is its input position, so the encoder
// stores inverse[bag] = segment directly. Any other batch holds many
// lookups per key (a multi-hot batch: 78 M lookups of 5.7 M keys in the
// 100-table workload), so the encoder writes one entry per segment into a
// map from key to segment, and k_inverse reads each lookup's key in input
// order and gathers its segment: coalesced stores and mostly cached gathers
// in place of one scattered 4-byte store per lookup.
//
// A segment starts where the key changes. A chunk starts at every segment
// start and at every multiple of kChunk sorted positions, so every chunk lies
// in one segment and in one kChunk-tile; a segment longer than a tile (a
// Zipf-hot key) is thereby split into pieces that can be reduced in parallel
// and combined in a fixed order. Three running quantities are scanned in one
// pass (count per tile, scan of tile counts, write): the number of segment
// starts, the number of chunk starts, and the position of the latest segment
// start (a max-scan). With them, the last position of every chunk writes the
// chunk's whole descriptor -- start, end, key, segment, and whether it is the
// entire segment -- so the reduce kernel needs a single 16-byte load per
// chunk.
#include "emb_device.h"

namespace emb {

__device__ __forceinline__ uint32_t key_of(uint64_t x) { return (uint32_t)(x >> 32); }

// Inclusive max over the 64 lanes of a wave, lane order.
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(v, d, 64);
    if (lane >= d) v = max(v, y);
  }
  return v;
}

// Per tile: segment starts, chunk starts, 1 + the last segment start in the
// tile (0 if none), and whether the key-build groups of this tile's share
// (32 groups of 64 bags) all hold one lookup per bag at the bag's own index.
__global__ __launch_bounds__(256) void k_rle_count(const uint64_t* __restrict__ sorted, int N,
                                                   const int32_t* __restrict__ unit_grp, int ngrp,
                                                   u4* __restrict__ blk_out) {
  __shared__ uint32_t lds[8];
  __shared__ uint32_t s_max[4];
  const long long base = (long long)blockIdx.x * kSortTile;
  // every item's key and its predecessor's are loaded first, from the tile's
  // start (a scalar base) at clamped 32-bit offsets: no branch and few
  // address registers, so the loads go out back to back
  uint32_t kc[kSortIPT], kp[kSortIPT];
  const int lim = (int)min((long long)N - base, (long long)kSortTile) - 1;  // >= 0: the grid covers [0, N)
  const uint64_t* tb = sorted + base;
  const int pmin = base > 0 ? -1 : 0;  // the word before the tile, if there is one
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const int o = min(k * 256 + (int)threadIdx.x, lim);
    kc[k] = key_of(tb[o]);
    kp[k] = key_of(tb[max(o - 1, pmin)]);
  }
  uint32_t cs = 0, cc = 0, ms = 0;
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 256 + threadIdx.x;
    if (i < N) {
      const bool fs = i == 0 || kc[k] != kp[k];
      const bool fc = fs || (i % kChunk) == 0;
      cs += fs;
      cc += fc;
      if (fs) ms = max(ms, (uint32_t)i + 1u);
    }
  }
  uint32_t ts, tc;
  block_excl_scan_256(cs, lds, &ts);
  block_excl_scan_256(cc, lds, &tc);
  uint32_t unit = 0;
  if (ngrp > 0) {  // uniform over the grid
    constexpr int kGrp = kSortTile / 64;
    const int gi = (int)blockIdx.x * kGrp + (int)threadIdx.x;
    unit = (uint32_t)__syncthreads_and((int)threadIdx.x >= kGrp || gi >= ngrp || unit_grp[gi] != 0);
  }
  const uint32_t wm = wave_incl_max(ms);
  if ((threadIdx.x & 63) == 63) s_max[threadIdx.x >> 6] = wm;
  __syncthreads();
  if (threadIdx.x == 0)
    blk_out[blockIdx.x] = u4{ts, tc, max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3])), unit};
}

// One block: exclusive scans of the per-tile counts (sum) and of the last
// segment start (max), in place; totals to *num_unique and num_chunks. Every
// entry's 4th word becomes 1 if all tiles reported one lookup per bag at
// the bag's own index (then the bag of position p is p).
__global__ __launch_bounds__(256) void k_rle_scan(u4* __restrict__ blk, int nblk,
                                                  int32_t* __restrict__ num_unique,
                                                  int32_t* __restrict__ num_chunks) {
  __shared__ uint32_t lds[8];
  __shared__ uint32_t s_max[4];
  // thread t owns tiles [t*per, (t+1)*per), read 8 at a time
  const int per = (nblk + 255) / 256;
  const int b0 = threadIdx.x * per;
  const int b1 = min(b0 + per, nblk);
  uint32_t ss = 0, sc = 0, sm = 0, su = 1;
  for (int i0 = b0; i0 < b1; i0 += 8) {
    u4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = i0 + k < b1 ? blk[i0 + k] : u4{0u, 0u, 0u, 1u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ss += v[k].x;
      sc += v[k].y;
      sm = max(sm, v[k].z);
      su &= v[k].w;
    }
  }
  const uint32_t unit = (uint32_t)__syncthreads_and((int)su);
  uint32_t ts, tc;
  uint32_t ps = block_excl_scan_256(ss, lds, &ts);
  uint32_t pc = block_excl_scan_256(sc, lds, &tc);
  // exclusive max over threads (thread order = tile order)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_max(sm);
  uint32_t pm = __shfl_up(incl, 1, 64);
  if (lane == 0) pm = 0;
  if (lane == 63) s_max[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) pm = max(pm, s_max[w]);
  for (int i0 = b0; i0 < b1; i0 += 8) {
    u4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = i0 + k < b1 ? blk[i0 + k] : u4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (i0 + k < b1) blk[i0 + k] = u4{ps, pc, pm, unit};
      ps += v[k].x;
      pc += v[k].y;
      pm = max(pm, v[k].z);
    }
  }
  if (threadIdx.x == 0) {
    *num_unique = (int32_t)ts;
    *num_chunks = (int32_t)tc;
  }
}

struct RleArgs {
  const uint64_t* sorted;
  const u4* blk;
  int32_t* seg_of_key;  // [total_rows + T] (batches that are not one lookup per bag)
  uint32_t total_rows;
  int B;
  uint32_t* unique_keys;
  int32_t* inverse;
  int32_t* seg_off;
  int4* desc;
  int32_t* counts;
  int32_t* chunk_seg;
  int32_t* tile_first_seg;
  int32_t* tile_last_seg;
  int32_t* sorted_bag;
  int N;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_rle_write(RleArgs a) {
  __shared__ uint32_t s_ws[4], s_wc[4], s_wm[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const long long base = (long long)blockIdx.x * kSortTile + wave * (64 * kSortIPT);
  const uint64_t le = lanemask_lt() | (1ull << lane);
  uint64_t item[kSortIPT];
  uint32_t is[kSortIPT], ic[kSortIPT], im[kSortIPT];
  uint32_t fl = 0;  // bit k: segment start, 8+k: chunk start, 16+k: segment end, 24+k: chunk end
  uint32_t run_s = 0, run_c = 0, run_m = 0;
  // The wave's 64 * kSortIPT consecutive words are loaded first, at clamped
  // indices (no branch: the loads go out back to back), plus the word before
  // and the word after the wave's range; every other neighbour's key comes
  // from the lane next to it (or the previous / next item's end lane).
  // (scalar wave base, 32-bit offsets: few address registers)
  const long long wbase = __builtin_amdgcn_readfirstlane((int)(base - (long long)blockIdx.x * kSortTile)) +
                          (long long)blockIdx.x * kSortTile;
  const int wlim = (int)max(min((long long)a.N - wbase, (long long)(64 * kSortIPT)), 1ll) - 1;
  const uint64_t* wb = a.sorted + min(wbase, (long long)a.N - 1);
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) item[k] = wb[min(k * 64 + lane, wlim)];
  const uint32_t key_before = key_of(wbase > 0 ? a.sorted[min(wbase - 1, (long long)a.N - 1)] : 0ull);
  const uint32_t key_after = key_of(a.sorted[min(wbase + 64 * kSortIPT, (long long)a.N - 1)]);
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 64 + lane;
    const uint32_t key = key_of(item[k]);
    const uint32_t up = (uint32_t)__shfl_up((int)key, 1, 64);
    const uint32_t dn = (uint32_t)__shfl_down((int)key, 1, 64);
    const uint32_t end_prev = (uint32_t)__builtin_amdgcn_readlane((int)key_of(item[k > 0 ? k - 1 : 0]), 63);
    const uint32_t start_next =
        (uint32_t)__builtin_amdgcn_readlane((int)key_of(item[k < kSortIPT - 1 ? k + 1 : k]), 0);
    const uint32_t kprev = lane > 0 ? up : (k > 0 ? end_prev : key_before);
    const uint32_t knext = lane < 63 ? dn : (k < kSortIPT - 1 ? start_next : key_after);
    bool fs = false, fc = false, se = false, ce = false;
    if (i < a.N) {
      fs = i == 0 || key != kprev;
      fc = fs || (i % kChunk) == 0;
      se = i + 1 == a.N || key != knext;
      ce = se || ((i + 1) % kChunk) == 0;
    } else {
      item[k] = 0;
    }
    const uint64_t bs = __ballot(fs);
    const uint64_t bc = __ballot(fc);
    is[k] = run_s + (uint32_t)__popcll(bs & le);
    ic[k] = run_c + (uint32_t)__popcll(bc & le);
    run_s += (uint32_t)__popcll(bs);
    run_c += (uint32_t)__popcll(bc);
    const uint32_t m = wave_incl_max(fs ? (uint32_t)i + 1u : 0u);
    im[k] = max(run_m, m);
    run_m = max(run_m, (uint32_t)__shfl(m, 63, 64));
    fl |= (fs ? 1u << k : 0u) | (fc ? 1u << (8 + k) : 0u) | (se ? 1u << (16 + k) : 0u) |
          (ce ? 1u << (24 + k) : 0u);
  }
  if (lane == 0) {
    s_ws[wave] = run_s;
    s_wc[wave] = run_c;
    s_wm[wave] = run_m;
  }
  __syncthreads();
  const u4 bp = a.blk[blockIdx.x];
  uint32_t ps = bp.x, pc = bp.y, pm = bp.z;
  for (int w = 0; w < wave; ++w) {
    ps += s_ws[w];
    pc += s_wc[w];
    pm = max(pm, s_wm[w]);
  }
  // one lookup per bag at the bag's own index (one-hot features): a word's
  // bag is its input position, and the inverse is stored directly
  const bool unit = bp.w != 0u;
  const uint64_t* __restrict__ sorted = a.sorted;
  int32_t bag[kSortIPT], cbv[kSortIPT], bag0[kSortIPT];
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 64 + lane;
    bag[k] = i < a.N ? (int32_t)(uint32_t)item[k] : -1;
    // chunk start: the later of its segment's start and its tile's start
    const int32_t seg_start = (int32_t)max(pm, im[k]) - 1;
    const int32_t tile0 = (int32_t)((i / kChunk) * kChunk);
    cbv[k] = seg_start > tile0 ? seg_start : tile0;
  }
  // the bag of each chunk's first lookup (loads first, stores after, so the
  // loads of all items are in flight together)
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 64 + lane;
    bag0[k] = bag[k];
    if (i < a.N && (fl & (1u << (24 + k))) && cbv[k] != (int32_t)i) bag0[k] = (int32_t)(uint32_t)sorted[cbv[k]];
  }
#pragma unroll
  for (int k = 0; k < kSortIPT; ++k) {
    const long long i = base + k * 64 + lane;
    if (i >= a.N) continue;
    const int32_t seg = (int32_t)(ps + is[k] - 1);
    const int32_t chk = (int32_t)(pc + ic[k] - 1);
    const int32_t seg_start = (int32_t)max(pm, im[k]) - 1;
    const uint32_t key = key_of(item[k]);
    if (unit) {
      // the inverse index with ordinary stores: the 4-byte stores of nearby
      // positions (a hot key's, or a tile's neighbours on one XCD) merge in
      // L2 before a line is written back
      if ((uint32_t)bag[k] < (uint32_t)a.N) a.inverse[bag[k]] = seg;
    } else if (key < a.total_rows) {
      if (fl & (1u << k)) a.seg_of_key[key] = seg;
    } else {
      // lookups with out-of-range indices: each table's sentinel entry gets
      // the segment of the run holding them (one run per table, or one run
      // for all tables when the sort ran over the whole key)
      a.seg_of_key[(size_t)a.total_rows + (uint32_t)bag[k] / (uint32_t)a.B] = seg;
    }
    // the sorted bags are written whole lines at a time: non-temporal, so they
    // keep the L2 for the forward / update running beside the dedup
    __builtin_nontemporal_store(bag[k], a.sorted_bag + i);
    if (fl & (1u << k)) {
      a.unique_keys[seg] = key;
      a.seg_off[seg] = (int32_t)i;
    }
    if (fl & (1u << (16 + k))) a.counts[seg] = (int32_t)i + 1 - seg_start;  // segment end
    if ((i % kChunk) == 0) a.tile_first_seg[i / kChunk] = seg;
    if ((i % kChunk) == kChunk - 1 || i == a.N - 1) a.tile_last_seg[i / kChunk] = seg;
    if (i == a.N - 1) a.seg_off[seg + 1] = a.N;
    if (fl & (1u << (24 + k))) {
      // last position of chunk `chk`; it is the whole segment when it starts
      // at the segment start and ends at the segment end. The descriptor also
      // carries the bag of the chunk's first lookup, so a one-lookup chunk
      // needs no further index load in the reduce kernel.
      const bool whole = cbv[k] == seg_start && (fl & (1u << (16 + k)));
      a.desc[chk] = int4{cbv[k], (int32_t)((uint32_t)(i + 1) | (whole ? 0x80000000u : 0u)), (int32_t)key, bag0[k]};
      a.chunk_seg[chk] = seg;
    }
  }
}

// inverse[i] = segment of lookup i's key, from the key -> segment map the
// encoder wrote (batches that are not one lookup per bag; the flag is the
// encoder's, uniform over the grid).
__global__ __launch_bounds__(256) void k_inverse(const u4* __restrict__ blk, const uint32_t* __restrict__ key_of_pos,
                                                 const int32_t* __restrict__ seg_of_key, uint32_t map_size, int N,
                                                 int32_t* __restrict__ inverse) {
  if (blk[0].w != 0u) return;  // one lookup per bag: stored by the encoder
  const long long i0 = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= N) return;
  // a whole group of 4 is one 16-byte load and (when `inverse` is 16-byte
  // aligned) one 16-byte store: four guarded stores would each end a basic
  // block, and each would wait for the ones before it
  const bool whole = i0 + 4 <= N;
  uint32_t k[4];
  if (whole) {
    const u4 kv = __builtin_nontemporal_load(reinterpret_cast<const u4*>(key_of_pos + i0));
    k[0] = kv.x;
    k[1] = kv.y;
    k[2] = kv.z;
    k[3] = kv.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = i0 + j < N ? key_of_pos[i0 + j] : map_size;
  }
  int32_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = k[j] < map_size ? seg_of_key[k[j]] : -1;
  if (whole && (reinterpret_cast<uintptr_t>(inverse) & 15u) == 0) {
    *reinterpret_cast<u4*>(inverse + i0) = u4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + j < N) inverse[i0 + j] = v[j];
  }
}

__global__ void k_set_empty(int32_t* num_unique, int32_t* num_chunks) {
  if (threadIdx.x == 0) {
    *num_unique = 0;
    *num_chunks = 0;
  }
}

hipError_t launch_rle(const Geom& g, int B, const uint64_t* sorted, int N, int ngrp, const WsLayout& L, char* ws,
                      const RleOut& o, hipStream_t st) {
  u4* blk = reinterpret_cast<u4*>(ws + L.rle_blk);
  int32_t* num_chunks = reinterpret_cast<int32_t*>(ws + L.scalars);
  const int nblk = L.nblk_rle;
  hipLaunchKernelGGL(k_rle_count, dim3(nblk), dim3(256), 0, st, sorted, N,
                     reinterpret_cast<const int32_t*>(ws + L.unit_grp), ngrp, blk);
  hipLaunchKernelGGL(k_rle_scan, dim3(1), dim3(256), 0, st, blk, nblk, o.num_unique, num_chunks);
  RleArgs a;
  a.sorted = sorted;
  a.blk = blk;
  a.seg_of_key = reinterpret_cast<int32_t*>(ws + L.seg_of_key);
  a.total_rows = g.total_rows;
  a.B = B > 0 ? B : 1;
  a.unique_keys = o.unique_keys;
  a.inverse = o.inverse;
  a.seg_off = reinterpret_cast<int32_t*>(ws + L.seg_off);
  a.desc = reinterpret_cast<int4*>(ws + L.desc);
  a.counts = o.counts;
  a.chunk_seg = reinterpret_cast<int32_t*>(ws + L.chunk_seg);
  a.tile_first_seg = reinterpret_cast<int32_t*>(ws + L.tile_first_seg);
  a.tile_last_seg = reinterpret_cast<int32_t*>(ws + L.tile_last_seg);
  a.sorted_bag = reinterpret_cast<int32_t*>(ws + L.sorted_bag);
  a.N = N;
  hipLaunchKernelGGL(k_rle_write, dim3(nblk), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_inverse, dim3(ceil_div(N, 1024)), dim3(256), 0, st, blk,
                     reinterpret_cast<const uint32_t*>(ws + L.key_of_pos), a.seg_of_key,
                     g.total_rows + (uint32_t)g.T, N, o.inverse);
  return hipGetLastError();
}

hipError_t launch_set_empty(const WsLayout& L, char* ws, int32_t* num_unique, hipStream_t st) {
  hipLaunchKernelGGL(k_set_empty, dim3(1), dim3(64), 0, st, num_unique,
                     reinterpret_cast<int32_t*>(ws + L.scalars));
  return hipGetLastError();
}

}  // namespace emb
