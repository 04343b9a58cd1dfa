// Backward, gradient side: per-key segmented gradient reduction and the
// sparse optimizer step, fused.
//
// For unique key u (segment [seg_off[u], seg_off[u+1]) of the sorted
// lookups) the gradient of its row is
//   g_u = sum_{i in segment} scale_i * dY[b(i)][t*D .. t*D+D),  scale_i = 1 or 1/L,
// the dense scatter-add of the per-lookup gradients restricted to the row
// (EMBark's reduction-based compression applied locally: one reduced gradient
// per distinct key). The optimizer then runs once per unique row, in fp32
// ("Merlin HugeCTR" GTC 2022 deck, slide "WEIGHT CONVERSION FOR MIXED
// PRECISION TRAINING": the optimizer computes in FP32):
//   SGD:     w <- w - (lr*g)
//   Adagrad: G <- G + g*g;  w <- w - (lr*g) / (sqrt(G) + eps)
// each operation rounded separately (no contraction), and w rounded back to
// the storage type with round-to-nearest-even. A low-precision table with an
// fp32 master (the same slide: FP32 master weights cast to the low-precision
// weights) steps the master instead and writes the master and its RNE cast in
// the same pass; its stored copy is never read here. Rows no lookup touched
// are never read or written.
//
// Work split. Segments are cut into chunks (at segment starts and every
// kChunk sorted positions). One subgroup of LPR lanes (4 fp32 columns per
// lane, so a dY row is one coalesced access; rows wider than a wave's 256
// columns take two column blocks on the grid's y axis) reduces one chunk,
// keeping 4 to 6 dY rows in flight (as many as fit 64 VGPRs without spills).
// On multi-hot batches a run of equal bags inside a segment loads its dY row
// once and reuses it. A chunk that is a whole segment
// applies the optimizer right there, with the weight (and state) row
// prefetched before the dY loop, so the reduced gradient never leaves VGPRs.
// A segment longer than a tile leaves one partial per kChunk-tile it touches
// (at most two partial slots per tile). k_level1 adds them per kChunk1-tile,
// and k_combine adds what the segment needs (level-0 partials inside one
// kChunk1-tile, else the level-1 ones) in tile order -- a fixed order, so
// results are bit-reproducible run to run -- and applies the update. No
// atomics touch gradients or weights.
#include "emb_device.h"

namespace emb {

struct RedArgs {
  const int32_t* sorted_bag;
  const float* inv_len;  // 1/L per bag, mean pooling only
  const float* dY;
  const uint32_t* ukeys;
  const int32_t* seg_off;
  const int4* desc;
  const int32_t* chunk_seg;
  const int32_t* num_chunks;
  const int32_t* num_unique;
  const int32_t* tile_first_seg;
  const int32_t* tile_last_seg;
  float* partial0;
  float* partial1;
  float* grad;  // reduced gradient out (mode 0) or in (apply)
  const int32_t* slot;  // mode 0: row of grad for segment u (null = u; < 0 = none)
  const DevTable* tables;
  const uint32_t* row_off;
  int T, B, D, Dsl;
  uint32_t total_rows;
  int N;
  int ntiles, ntiles1;
  float lr, eps;
  int ptr_lds;  // k_chunks: the tables' row pointers (one slice each) are staged in LDS
};

// DT below is the update type code: storage type, | kMasterBit with a master.
template <int DT>
__device__ __forceinline__ void row_ptrs(const RedArgs& a, int t, uint32_t r, int c0, char** wp,
                                         float** gp, float** mp) {
  const int s = c0 / a.Dsl;
  const int cs = c0 - s * a.Dsl;
  const size_t e = (size_t)r * a.Dsl + cs;
  *wp = reinterpret_cast<char*>(a.tables[t].w[s]) + e * Stor<(DT & 7)>::kBytes;
  float* g = a.tables[t].g[s];
  *gp = g ? g + e : nullptr;
  if constexpr ((DT & kMasterBit) != 0) *mp = a.tables[t].m[s] + e;
}

// The fp32 value the optimizer steps: the master if there is one, else the
// widened stored weight.
template <int DT>
__device__ __forceinline__ void load_weight(const char* wp, const float* mp, float* wv) {
  if constexpr ((DT & kMasterBit) != 0)
    load4<EMB_F32>(mp, wv);
  else
    load4<(DT & 7)>(wp, wv);
}

// mode 1 = SGD, 2 = Adagrad
template <int DT, int MODE>
__device__ __forceinline__ void row_update(char* wp, float* gp, float* mp, const float* wv,
                                           const float* Gv, const float* g, float lr, float eps) {
#pragma clang fp contract(off)
  float nw[4];
  if constexpr (MODE == 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) nw[c] = wv[c] - lr * g[c];
  } else {
    float ng[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ng[c] = Gv[c] + g[c] * g[c];
      const float den = __fsqrt_rn(ng[c]) + eps;
      nw[c] = wv[c] - __fdiv_rn(lr * g[c], den);
    }
    f4 v = {ng[0], ng[1], ng[2], ng[3]};
    *reinterpret_cast<f4*>(gp) = v;
  }
  if constexpr ((DT & kMasterBit) != 0) {
    f4 m = {nw[0], nw[1], nw[2], nw[3]};
    *reinterpret_cast<f4*>(mp) = m;
  }
  store4<(DT & 7)>(wp, nw);
}

// Applies the finished gradient of unique key `key` (segment `seg`): mode 0
// stores it, modes 1/2 run the optimizer on the row.
template <int DT, int MODE>
__device__ __forceinline__ void finish_row(const RedArgs& a, const uint32_t* s_ro, uint32_t key,
                                           int seg, int c0, const float* g) {
  if constexpr (MODE == 0) {
    const int dst = a.slot ? a.slot[seg] : seg;
    if ((unsigned)dst < (unsigned)a.N) {
      f4 o = {g[0], g[1], g[2], g[3]};
      *reinterpret_cast<f4*>(a.grad + (size_t)dst * a.D + c0) = o;
    }
  } else {
    const int t = table_of(s_ro, a.T, key);
    char* wp;
    float* gp;
    float* mp = nullptr;
    row_ptrs<DT>(a, t, key - s_ro[t], c0, &wp, &gp, &mp);
    float wv[4], Gv[4] = {0.f, 0.f, 0.f, 0.f};
    load_weight<DT>(wp, mp, wv);
    if constexpr (MODE == 2) load4<EMB_F32>(gp, Gv);
    row_update<DT, MODE>(wp, gp, mp, wv, Gv, g, a.lr, a.eps);
  }
}

// Level-0 slot of the partial sum of segment [so, eo) in tile j: the chunk of
// the segment in tile j starts at the tile start (slot 2j) unless the
// segment itself starts inside tile j (slot 2j+1). Same rule at level 1.
__device__ __forceinline__ int slot_of(int so, int j, int tile) {
  return (j == so / tile && so % tile != 0) ? 2 * j + 1 : 2 * j;
}

// REP: the batch may hold a key more than once in one bag (more lookups than
// bags), so a segment can repeat a bag; see the multi-hot loop below.
template <int DT, int LPR, int MODE, bool MEAN, bool REP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_chunks(RedArgs a) {
  // With ptr_lds (multi-hot batches of unsliced tables, few of them) the tables' weight, state and
  // master pointers sit in LDS ahead of the row offsets, so a chunk's row
  // address needs no global load of its table's descriptor: the weight and
  // state loads go out with the dY loads.
  extern __shared__ uint64_t s_dyn[];
  const bool ptr_lds = REP && a.ptr_lds;  // set only for multi-hot batches
  const int nptr = ptr_lds ? 3 * a.T : 0;
  char** s_w = reinterpret_cast<char**>(s_dyn);
  float** s_g = reinterpret_cast<float**>(s_dyn + a.T);
  float** s_m = reinterpret_cast<float**>(s_dyn + 2 * a.T);
  uint32_t* s_ro = reinterpret_cast<uint32_t*>(s_dyn + nptr);
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  for (int i = threadIdx.x; i < (ptr_lds ? a.T : 0); i += 256) {
    s_w[i] = reinterpret_cast<char*>(a.tables[i].w[0]);
    s_g[i] = a.tables[i].g[0];
    s_m[i] = a.tables[i].m[0];
  }
  __syncthreads();
  // dY rows in flight: the largest count that fits 64 VGPRs without spills at
  // 8 waves/SIMD (spills cost scratch traffic in HBM: measured ~270 MB/launch);
  // Adagrad with mean pooling or a 16-bit / master row holds more live values
  constexpr int U0 = (MODE == 2 && (MEAN || (DT & 7) != EMB_F32 || (DT & kMasterBit))) ? 4 : 6;
  // multi-hot: the next group's bags take registers too (fp32 Adagrad rows
  // then fit 4 in flight without spills)
  constexpr int U = REP ? (MODE == 2 && U0 == 6 ? 4 : U0 - 1) : U0;
  constexpr int SGW = 256 / LPR;
  const int lsg = threadIdx.x & (LPR - 1);
  // blockIdx.y picks the column block: rows wider than 4*LPR columns
  // (16-bit rows of more than 256) are spread over gridDim.y blocks
  const int c0 = (int)blockIdx.y * 4 * LPR + lsg * 4;
  const bool act = c0 < a.D;
  const uint32_t dys = (uint32_t)(a.T * a.D);
  const int nsg = gridDim.x * SGW;
  const int nch = min(*a.num_chunks, a.N + a.ntiles);
  int q = blockIdx.x * SGW + threadIdx.x / LPR;
  // The next descriptor is loaded while the current chunk is processed. The
  // subgroups of a wave take consecutive chunks, so with at most 2 per wave
  // (LPR >= 32) the wave reads its next 2 descriptors with scalar loads from a
  // uniform base: those are counted apart from the vector loads, so the waits
  // for dY and row loads never wait for them. The base is clamped so that
  // [qb, qb + W) stays inside the buffer (N + ntiles + 4 entries); a subgroup
  // past the list's end picks a duplicate it never uses. The pick happens
  // where the loop moves on, and the loads are issued after the chunk's last
  // LDS read (LDS and scalar loads share a wait counter). Narrower subgroups
  // load their next descriptor with a vector load at the loop's head.
  constexpr int W = 64 / LPR;
  constexpr bool kScalarDesc = W <= 2;
  typedef const __attribute__((address_space(4))) int* cdesc_t;
  const int sub_in_wave = (int)(threadIdx.x & 63) / LPR;
  int4 vn0 = {0, 0, -1, -1}, vn1 = {0, 0, -1, -1};
  int qbn = 0;
  auto prefetch = [&](int qn) {
    if constexpr (kScalarDesc) {
      int qb = __builtin_amdgcn_readfirstlane(qn - sub_in_wave);
      qb = max(min(qb, nch - W), 0);
      const cdesc_t p = (cdesc_t)(a.desc) + 4 * qb;
      vn0 = int4{p[0], p[1], p[2], p[3]};
      if constexpr (W == 2) vn1 = int4{p[4], p[5], p[6], p[7]};
      qbn = qb;
    }
  };
  int4 d = q < nch ? a.desc[q] : int4{0, 0, -1, -1};
  for (; q < nch; q += nsg, d = (kScalarDesc && q - qbn == 1) ? vn1 : vn0) {
    if constexpr (!kScalarDesc) vn0 = a.desc[min(q + nsg, nch - 1)];
    // every index below is clamped into its buffer: a wrong count or offset
    // can give a wrong result, never an access outside the workspace
    const int cb = max(d.x, 0);
    const int ce = min(d.y & 0x7fffffff, a.N);
    const bool whole = d.y < 0;
    const uint32_t key = (uint32_t)d.z;
    const int bag0 = d.w;
    if (key >= a.total_rows) {  // lookups with out-of-range indices
      prefetch(q + nsg);
      continue;
    }
    const int t = table_of(s_ro, a.T, key);

    char* wp = nullptr;
    float* gp = nullptr;
    float* mp = nullptr;
    float wv[4] = {0.f, 0.f, 0.f, 0.f}, Gv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE != 0) {
      if (whole && act) {  // prefetch the row so its latency overlaps the dY loads
        if (ptr_lds) {
          const size_t e = (size_t)(key - s_ro[t]) * a.D + c0;
          wp = s_w[t] + e * Stor<(DT & 7)>::kBytes;
          gp = s_g[t] ? s_g[t] + e : nullptr;
          if constexpr ((DT & kMasterBit) != 0) mp = s_m[t] + e;
        } else {
          row_ptrs<DT>(a, t, key - s_ro[t], c0, &wp, &gp, &mp);
        }
        load_weight<DT>(wp, mp, wv);
        if constexpr (MODE == 2) load4<EMB_F32>(gp, Gv);
      }
    }
    // the chunk's last LDS read is behind: issue the next descriptor now
    prefetch(q + nsg);

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    // dY element offsets fit in 32 bits (fewer than 2^32 elements), so the
    // loads use the uniform base + a 32-bit per-lane offset
    const uint32_t dyt = (uint32_t)(t * a.D + c0);
    const int bagt = t * a.B;
    if constexpr (REP) {
      // Multi-hot: a chunk can run to kChunk positions. The bags of the next
      // U positions are loaded while this group's dY rows are in flight, so
      // an iteration waits one memory round trip, not two. A segment's
      // positions are ascending, so repeats of one bag (a key looked up
      // several times in one bag) sit next to each other: a run's first
      // entry loads the row and the others reuse it. Entries are added one
      // by one in position order, so the sum does not depend on U (the fused
      // and the materialised paths, whose U differ, agree bit for bit).
      int bn[U];
#pragma unroll
      for (int k = 0; k < U; ++k) bn[k] = cb + k < ce ? (k == 0 ? bag0 : a.sorted_bag[cb + k]) : -1;
      for (int i = cb; i < ce; i += U) {
        int bg[U];
#pragma unroll
        for (int k = 0; k < U; ++k) bg[k] = bn[k];
        f4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          v[k] = f4{0.f, 0.f, 0.f, 0.f};
          const unsigned b = (unsigned)(bg[k] - bagt);
          if (bg[k] >= 0 && b < (unsigned)a.B && act && (k == 0 || bg[k] != bg[k - 1])) {
            v[k] = *reinterpret_cast<const f4*>(a.dY + (b * dys + dyt));
            if constexpr (MEAN) v[k] *= a.inv_len[bg[k]];
          }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) bn[k] = i + U + k < ce ? a.sorted_bag[i + U + k] : -1;
#pragma unroll
        for (int k = 1; k < U; ++k)
          if (bg[k] >= 0 && bg[k] == bg[k - 1]) v[k] = v[k - 1];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          acc[0] += v[k].x;
          acc[1] += v[k].y;
          acc[2] += v[k].z;
          acc[3] += v[k].w;
        }
      }
    } else {
      for (int i = cb; i < ce; i += U) {
        int bg[U];
#pragma unroll
        for (int k = 0; k < U; ++k) bg[k] = i + k < ce ? (i + k == cb ? bag0 : a.sorted_bag[i + k]) : -1;
        f4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          v[k] = f4{0.f, 0.f, 0.f, 0.f};
          const unsigned b = (unsigned)(bg[k] - bagt);
          if (bg[k] >= 0 && b < (unsigned)a.B && act) {
            v[k] = *reinterpret_cast<const f4*>(a.dY + (b * dys + dyt));
            if constexpr (MEAN) v[k] *= a.inv_len[bg[k]];
          }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
          acc[0] += v[k].x;
          acc[1] += v[k].y;
          acc[2] += v[k].z;
          acc[3] += v[k].w;
        }
      }
    }

    if (!act) continue;
    if (whole) {
      if constexpr (MODE == 0) {
        const int seg = a.chunk_seg[q];
        if ((unsigned)seg < (unsigned)a.N) {
          const int dst = a.slot ? a.slot[seg] : seg;
          if ((unsigned)dst < (unsigned)a.N) {
            f4 o = {acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f4*>(a.grad + (size_t)dst * a.D + c0) = o;
          }
        }
      } else {
        row_update<DT, MODE>(wp, gp, mp, wv, Gv, acc, a.lr, a.eps);
      }
    } else {
      const int j = cb / kChunk;
      const int slot = 2 * j + (cb == j * kChunk ? 0 : 1);
      f4 o = {acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f4*>(a.partial0 + (size_t)slot * a.D + c0) = o;
    }
  }
}

// Sums `n` partial rows partial[slot(k)], k = 0..n-1, in k order, 8 in flight.
template <typename SlotFn>
__device__ __forceinline__ void sum_partials(const float* partial, int D, int c0, bool act, int n,
                                             SlotFn slot, float* g) {
  constexpr int U = 8;
  g[0] = g[1] = g[2] = g[3] = 0.f;
  for (int k0 = 0; k0 < n; k0 += U) {
    f4 v[U];
#pragma unroll
    for (int m = 0; m < U; ++m) {
      v[m] = f4{0.f, 0.f, 0.f, 0.f};
      if (k0 + m < n && act) v[m] = *reinterpret_cast<const f4*>(partial + (size_t)slot(k0 + m) * D + c0);
    }
#pragma unroll
    for (int m = 0; m < U; ++m) {
      g[0] += v[m].x;
      g[1] += v[m].y;
      g[2] += v[m].z;
      g[3] += v[m].w;
    }
  }
}

// Level 1: two subgroups per 4096-position tile J. The segments that cross
// a level-1 boundary and touch J can only be J's first and last segments;
// subgroup c of J takes the first (c = 0) or the last (c = 1, unless it is
// the same segment) and adds its level-0 partials inside J (tile order) into
// its level-1 partial of J.
template <int LPR>
__global__ __launch_bounds__(256) void k_level1(RedArgs a) {
  constexpr int SGW = 256 / LPR;
  const int sgi = blockIdx.x * SGW + threadIdx.x / LPR;
  const int J = sgi >> 1;
  if (J >= a.ntiles1) return;
  const int c0 = (int)blockIdx.y * 4 * LPR + (threadIdx.x & (LPR - 1)) * 4;  // column block: blockIdx.y
  const bool act = c0 < a.D;
  const int jf = J * kL1Tiles;
  const int jl = min(jf + kL1Tiles - 1, a.ntiles - 1);
  const int first = a.tile_first_seg[jf];
  int u = first;
  if (sgi & 1) {
    u = a.tile_last_seg[jl];
    if (u == first) return;
  }
  if (u < 0 || u >= a.N || a.ukeys[u] >= a.total_rows) return;
  const int so = a.seg_off[u];
  const int eo = a.seg_off[u + 1];
  if (so / kChunk1 == (eo - 1) / kChunk1) return;  // stays inside one level-1 tile
  const int lo = max(so, J * kChunk1);
  const int hi = min(eo, (J + 1) * kChunk1);
  if (lo >= hi) return;
  const int j0 = lo / kChunk;
  const int n = (hi - 1) / kChunk - j0 + 1;
  float g[4];
  sum_partials(a.partial0, a.D, c0, act, n, [&](int k) { return slot_of(so, j0 + k, kChunk); }, g);
  const int slot1 = slot_of(so, J, kChunk1);
  if (act) {
    f4 o = {g[0], g[1], g[2], g[3]};
    *reinterpret_cast<f4*>(a.partial1 + (size_t)slot1 * a.D + c0) = o;
  }
}

// Final combine: one subgroup per level-0 tile j. It owns the segment that
// starts in tile j and runs past its end (at most one: the tile's last
// segment); it adds the segment's level-0 partials, or its level-1 partials if
// it crosses a level-1 boundary, in order, and applies the update.
template <int DT, int LPR, int MODE>
__global__ __launch_bounds__(256) void k_combine(RedArgs a) {
  constexpr int SGW = 256 / LPR;
  extern __shared__ uint32_t s_ro[];
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  __syncthreads();
  const int j = blockIdx.x * SGW + threadIdx.x / LPR;
  if (j >= a.ntiles) return;
  const int c0 = (int)blockIdx.y * 4 * LPR + (threadIdx.x & (LPR - 1)) * 4;  // column block: blockIdx.y
  const bool act = c0 < a.D;
  const int u = a.tile_last_seg[j];
  if (u < 0 || u >= a.N) return;
  const int so = a.seg_off[u];
  const int eo = a.seg_off[u + 1];
  if (so < j * kChunk || eo <= (j + 1) * kChunk) return;  // not the owner
  const uint32_t key = a.ukeys[u];
  if (key >= a.total_rows) return;
  // the row (and state) is loaded before the partials are summed, so its
  // latency overlaps theirs
  char* wp = nullptr;
  float* gp = nullptr;
  float* mp = nullptr;
  float wv[4] = {0.f, 0.f, 0.f, 0.f}, Gv[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE != 0) {
    if (act) {
      const int t = table_of(s_ro, a.T, key);
      row_ptrs<DT>(a, t, key - s_ro[t], c0, &wp, &gp, &mp);
      load_weight<DT>(wp, mp, wv);
      if constexpr (MODE == 2) load4<EMB_F32>(gp, Gv);
    }
  }
  float g[4];
  if (so / kChunk1 == (eo - 1) / kChunk1) {
    const int n = (eo - 1) / kChunk - j + 1;
    sum_partials(a.partial0, a.D, c0, act, n, [&](int k) { return slot_of(so, j + k, kChunk); }, g);
  } else {
    const int J0 = so / kChunk1;
    const int n = (eo - 1) / kChunk1 - J0 + 1;
    sum_partials(a.partial1, a.D, c0, act, n, [&](int k) { return slot_of(so, J0 + k, kChunk1); }, g);
  }
  if (!act) return;
  if constexpr (MODE == 0) finish_row<DT, MODE>(a, s_ro, key, u, c0, g);
  else row_update<DT, MODE>(wp, gp, mp, wv, Gv, g, a.lr, a.eps);
}

// Update from a materialised reduced gradient (grad[u] for u < U).
template <int DT, int LPR, int MODE>
__global__ __launch_bounds__(256) void k_apply(RedArgs a) {
  extern __shared__ uint32_t s_ro[];
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  __syncthreads();
  constexpr int SGW = 256 / LPR;
  const int lsg = threadIdx.x & (LPR - 1);
  const int c0 = (int)blockIdx.y * 4 * LPR + lsg * 4;  // column block: blockIdx.y
  if (c0 >= a.D) return;
  const int U = min(*a.num_unique, a.N);
  for (long long u = (long long)blockIdx.x * SGW + threadIdx.x / LPR; u < U;
       u += (long long)gridDim.x * SGW) {
    const uint32_t key = a.ukeys[u];
    if (key >= a.total_rows) continue;
    float g[4];
    load4<EMB_F32>(a.grad + (size_t)u * a.D + c0, g);
    finish_row<DT, MODE>(a, s_ro, key, (int)u, c0, g);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static RedArgs make_args(const Geom& g, const DevCtx& dc, int N, const WsLayout& L,
                         const char* ws, const uint32_t* ukeys, float lr, float eps) {
  RedArgs a;
  a.sorted_bag = reinterpret_cast<const int32_t*>(ws + L.sorted_bag);
  a.inv_len = nullptr;
  a.dY = nullptr;
  a.ukeys = ukeys;
  a.seg_off = reinterpret_cast<const int32_t*>(ws + L.seg_off);
  a.desc = reinterpret_cast<const int4*>(ws + L.desc);
  a.chunk_seg = reinterpret_cast<const int32_t*>(ws + L.chunk_seg);
  a.num_chunks = reinterpret_cast<const int32_t*>(ws + L.scalars);
  a.num_unique = nullptr;
  a.tile_first_seg = reinterpret_cast<const int32_t*>(ws + L.tile_first_seg);
  a.tile_last_seg = reinterpret_cast<const int32_t*>(ws + L.tile_last_seg);
  a.partial0 = const_cast<float*>(reinterpret_cast<const float*>(ws + L.partial0));
  a.partial1 = const_cast<float*>(reinterpret_cast<const float*>(ws + L.partial1));
  a.grad = nullptr;
  a.slot = nullptr;
  a.tables = dc.tables;
  a.row_off = dc.row_off;
  a.T = g.T;
  a.B = 0;
  a.D = g.D;
  a.Dsl = g.Dsl;
  a.total_rows = g.total_rows;
  a.N = N;
  a.ntiles = L.ntiles;
  a.ntiles1 = L.ntiles1;
  a.lr = lr;
  a.eps = eps;
  a.ptr_lds = 0;
  return a;
}

// Lanes per row for the fp32-gradient kernels: 4 columns per lane, at most a
// wave; wider rows take col_blocks() blocks along the grid's y axis.
static int lpr_b(const Geom& g) {
  int l = next_pow2((g.D + 3) / 4);
  return l < 2 ? 2 : (l > 64 ? 64 : l);
}

#define LPR_SWITCH(LAUNCH)          \
  switch (lpr) {                    \
    case 2: LAUNCH(2) break;        \
    case 4: LAUNCH(4) break;        \
    case 8: LAUNCH(8) break;        \
    case 16: LAUNCH(16) break;      \
    case 32: LAUNCH(32) break;      \
    default: LAUNCH(64) break;      \
  }

template <int DT, int MODE, bool MEAN, bool REP>
static void launch_chunks_t(int lpr, int grid, size_t smem, hipStream_t st, const RedArgs& a) {
#define L_CH(P) hipLaunchKernelGGL((k_chunks<DT, P, MODE, MEAN, REP>), dim3(grid, col_blocks(a.D, P)), dim3(256), smem, st, a);
  LPR_SWITCH(L_CH)
#undef L_CH
}

template <int DT, int MODE>
static void launch_combine_t(int lpr, int grid, size_t smem, hipStream_t st, const RedArgs& a) {
#define L_CO(P) hipLaunchKernelGGL((k_combine<DT, P, MODE>), dim3(grid, col_blocks(a.D, P)), dim3(256), smem, st, a);
  LPR_SWITCH(L_CO)
#undef L_CO
}

template <int DT, int MODE>
static void launch_apply_t(int lpr, int grid, size_t smem, hipStream_t st, const RedArgs& a) {
#define L_AP(P) hipLaunchKernelGGL((k_apply<DT, P, MODE>), dim3(grid, col_blocks(a.D, P)), dim3(256), smem, st, a);
  LPR_SWITCH(L_AP)
#undef L_AP
}

// Mode 0 (materialise the gradient) touches no weights, so it has one
// instantiation; modes 1/2 are instantiated per update type code.
#define DISPATCH_DT_MODE(FN, ...)                                                  \
  if (mode == 0) {                                                                 \
    FN<EMB_F32, 0>(__VA_ARGS__);                                                   \
  } else {                                                                         \
    switch (g.dtype | (g.master ? kMasterBit : 0)) {                               \
      case EMB_F32:                                                                \
        if (mode == 1) FN<EMB_F32, 1>(__VA_ARGS__);                                \
        else FN<EMB_F32, 2>(__VA_ARGS__);                                          \
        break;                                                                     \
      case EMB_BF16:                                                               \
        if (mode == 1) FN<EMB_BF16, 1>(__VA_ARGS__);                               \
        else FN<EMB_BF16, 2>(__VA_ARGS__);                                         \
        break;                                                                     \
      case EMB_F16:                                                                \
        if (mode == 1) FN<EMB_F16, 1>(__VA_ARGS__);                                \
        else FN<EMB_F16, 2>(__VA_ARGS__);                                          \
        break;                                                                     \
      case EMB_BF16 | kMasterBit:                                                  \
        if (mode == 1) FN<EMB_BF16 | kMasterBit, 1>(__VA_ARGS__);                  \
        else FN<EMB_BF16 | kMasterBit, 2>(__VA_ARGS__);                            \
        break;                                                                     \
      default:                                                                     \
        if (mode == 1) FN<EMB_F16 | kMasterBit, 1>(__VA_ARGS__);                   \
        else FN<EMB_F16 | kMasterBit, 2>(__VA_ARGS__);                             \
        break;                                                                     \
    }                                                                              \
  }

template <int DT, int MODE>
static void launch_chunks_pool(bool mean, bool rep, int lpr, int grid, size_t smem, hipStream_t st,
                               const RedArgs& a) {
  if (rep) {
    if (mean) launch_chunks_t<DT, MODE, true, true>(lpr, grid, smem, st, a);
    else launch_chunks_t<DT, MODE, false, true>(lpr, grid, smem, st, a);
  } else {
    if (mean) launch_chunks_t<DT, MODE, true, false>(lpr, grid, smem, st, a);
    else launch_chunks_t<DT, MODE, false, false>(lpr, grid, smem, st, a);
  }
}

hipError_t launch_reduce(const Geom& g, const DevCtx& dc, int mode, int N, int B, int pool,
                         const float* dY, const WsLayout& L, const char* ws,
                         const uint32_t* unique_keys, const int32_t* num_unique, float* grad_out,
                         float lr, float eps, hipStream_t st, const int32_t* slot) {
  RedArgs a = make_args(g, dc, N, L, ws, unique_keys, lr, eps);
  a.slot = slot;
  a.B = B;
  a.dY = dY;
  const bool mean = pool == EMB_POOL_MEAN;
  a.inv_len = mean ? reinterpret_cast<const float*>(ws + L.inv_len) : nullptr;
  a.num_unique = num_unique;
  a.grad = grad_out;
  const int lpr = lpr_b(g);
  const int sgw = 256 / lpr;
  // chunks <= N + ntiles; the loop is grid-strided over the device count
  const long long upper = (long long)N + L.ntiles;
  const long long want = (upper + sgw - 1) / sgw;
  // The grid is capped at one block per 32 bags, between 16384 and 32768
  // blocks: the chunk count grows with the bag count, and a longer chunk list
  // runs faster on the larger grid (26 x 4M x 128, 1.7 M bags: 437 -> 429 us;
  // 100 x 1M x 128 bf16, 3.3 M bags: 5.40 -> 5.16 ms beside the next dedup)
  // while a short one leaves its extra blocks idle (one 200M-row table, 65 k
  // bags: 90 -> 94 us).
  const long long bags = (long long)g.T * B;
  const long long cap = bags / 32 < 16384 ? 16384 : (bags / 32 > 32768 ? 32768 : bags / 32);
  const int grid = (int)(want < cap ? (want > 0 ? want : 1) : cap);
  // with no more lookups than bags a repeat is rare (it needs an empty bag
  // elsewhere); the plain loop is then the faster one, and both are exact
  const bool rep = (long long)N > (long long)g.T * B;
  // row pointers from LDS: measured faster on multi-hot batches (the
  // 100-table bf16 workload: 4.71 -> 4.64 ms) and no faster on one-hot ones
  // (26 x 4M x 128: 429.6 vs 430.8 us), so only there
  a.ptr_lds = rep && g.T <= 256 && g.Dsl == g.D ? 1 : 0;
  const size_t smem = (size_t)(a.ptr_lds ? 3 * g.T : 0) * 8 + (size_t)(g.T + 1) * 4;
  DISPATCH_DT_MODE(launch_chunks_pool, mean, rep, lpr, grid, smem, st, a)
  return hipGetLastError();
}

hipError_t launch_combine(const Geom& g, const DevCtx& dc, int mode, int N, const WsLayout& L,
                          const char* ws, const uint32_t* unique_keys, float* grad_out, float lr,
                          float eps, hipStream_t st, const int32_t* slot) {
  RedArgs a = make_args(g, dc, N, L, ws, unique_keys, lr, eps);
  a.slot = slot;
  a.grad = grad_out;
  const int lpr = lpr_b(g);
  const int sgw = 256 / lpr;
  if (L.ntiles1 > 1) {
    const int grid1 = ceil_div(2ll * L.ntiles1, sgw);  // two subgroups per level-1 tile
#define L_L1(P) hipLaunchKernelGGL((k_level1<P>), dim3(grid1, col_blocks(a.D, P)), dim3(256), 0, st, a);
    LPR_SWITCH(L_L1)
#undef L_L1
  }
  const int grid = ceil_div(L.ntiles, sgw);
  const size_t smem = (size_t)(g.T + 1) * 4;
  if (grid > 0) {
    DISPATCH_DT_MODE(launch_combine_t, lpr, grid, smem, st, a)
  }
  return hipGetLastError();
}

hipError_t launch_apply(const Geom& g, const DevCtx& dc, int mode, int N,
                        const uint32_t* unique_keys, const int32_t* num_unique,
                        const float* grad_in, float lr, float eps, hipStream_t st) {
  RedArgs a{};
  a.ukeys = unique_keys;
  a.num_unique = num_unique;
  a.grad = const_cast<float*>(grad_in);
  a.tables = dc.tables;
  a.row_off = dc.row_off;
  a.T = g.T;
  a.D = g.D;
  a.Dsl = g.Dsl;
  a.total_rows = g.total_rows;
  a.N = N;
  a.lr = lr;
  a.eps = eps;
  const int lpr = lpr_b(g);
  const int sgw = 256 / lpr;
  const long long want = ((long long)N + sgw - 1) / sgw;
  const int grid = (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
  const size_t smem = (size_t)(g.T + 1) * 4;
  DISPATCH_DT_MODE(launch_apply_t, lpr, grid, smem, st, a)
  return hipGetLastError();
}

}  // namespace emb
