// Pooled forward: multi-table, multi-hot lookup + sum/mean pooling +
// per-sample concatenation, in one kernel.
//
// What is computed follows "Merlin HugeCTR: GPU-accelerated recommender
// system training and inference" (GTC 2022 deck), slide "COMMON EMBEDDING
// PRIMITIVES" (table lookup, pooling/reduction of a multi-hot feature,
// concatenation) and slide "HUGECTR EMBEDDING LAYER" (lookup and in-register
// reduction + concatenation fused into one kernel): for bag (t, b),
//   out[b][t*D + c] = sum_{i in bag} W_t[idx_i][c]   (or / L for mean),
// accumulated in fp32 registers whatever the storage type.
//
// gfx950 mapping. A subgroup of LPR lanes owns one row: every lane loads 16
// bytes (4 fp32 or 8 bf16/fp16 columns), so a row is one coalesced
// LPR*16-byte access and a wave64 holds 64/LPR rows per load instruction.
// Each subgroup walks a run of `bps` consecutive bags of one table as one
// flat stream of lookups, issuing U = 4 row loads before consuming them, so
// one-hot bags (one row per bag) still keep 4 rows per subgroup in flight.
// The run's bag boundaries (bps+1 offsets) sit one per lane and are read by
// lane shuffles (ds_bpermute), not by dependent global loads; so do its row
// indices, LPR at a time and one block ahead, so that a row load waits on one
// round trip. Pooled rows
// are written with non-temporal stores so the L2 keeps Zipf-hot table rows.
// The grid may be capped (grid-stride over the work) so that the dedup, run
// on a second stream, keeps some wave slots while the forward streams.
//
// Unique-first variant (FLAT): after the step's keys are deduplicated, each
// unique row is gathered once into a compact [U][D] buffer (k_gather_unique)
// and the bags are pooled from it through the lookups' inverse indices -- the
// unique-based side of EMBark's compression (RecSys'24 article, embedding
// clusters) applied to the forward on one GPU's share.
#include "emb_device.h"

namespace emb {

struct FwdArgs {
  const void* indices;
  const void* offsets;
  const DevTable* tables;
  const uint32_t* row_off;
  float* out;
  int* err;
  long long N;
  int T, B, D, Dsl;
  int bps;           // bags per subgroup (<= LPR - 1)
  int sg_per_table;  // ceil(B / bps)
  long long total_sg;
  int nblk;
  int mean;
  const void* flat;    // SRC 1: the compact rows, [flat_rows][D] of the storage type,
                       // indexed by int32 `indices` (offsets stay of type IDX)
  long long flat_rows;
  const HashMeta* hmeta;        // SRC 2: `indices` are int64 ids looked up in
  unsigned long long* hkeys;    // the tables' hash maps (an id without a row
  const int* hvals;             // pools to nothing)
};

// 8 waves/SIMD with 4 rows in flight per subgroup measured faster than 5
// waves/SIMD with 8 rows (293 -> 277 us on the 26x4Mx128 one-hot workload).
// Positions are 32-bit (N < 2^31 is validated) to stay within 64 VGPRs.
// SRC: 0 = rows of the tables by index, 1 = compact unique rows by inverse,
// 2 = rows of the tables by hashed id (lookup only: the HugeCTR embedding
// layer's hash table lookup fused with the pooling).
// The hashed source needs more registers where a lane probes for 4 lookups
// (subgroups of 2 lanes) or widens 16-bit rows: 6 waves/SIMD there (no
// spills), 8 everywhere else.
template <int DT, typename IDX, int LPR, int SRC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    SRC == 2 && (LPR < 4 || DT != EMB_F32) ? 6 : 8, SRC == 2 && (LPR < 4 || DT != EMB_F32) ? 6 : 8))) void
k_forward(FwdArgs a) {
  constexpr int CPL = 16 / Stor<DT>::kBytes;  // columns per lane
  constexpr int SGW = 256 / LPR;              // subgroups per block
  constexpr int U = 4;                        // rows in flight per subgroup
  const int lsg = threadIdx.x & (LPR - 1);
  const int N = (int)a.N;
  // grid-stride over logical blocks: the grid may be capped below the work so
  // that kernels on another stream (the dedup) keep wave slots
  // With the full grid (padded to a multiple of 8) blocks are remapped so that
  // each XCD walks its own contiguous eighth of the bag runs: at any time an
  // XCD's L2 holds the hot rows of one table rather than every XCD holding
  // the same few tables' (HBM reads of the 26x4Mx128 one-hot forward: 468 ->
  // 384 MB per launch).
  const int blk_first =
      (gridDim.x & 7) == 0 && (int)gridDim.x >= a.nblk ? xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  for (int blk = blk_first; blk < a.nblk; blk += gridDim.x) {
    const long long sg = (long long)blk * SGW + threadIdx.x / LPR;
    if (sg >= a.total_sg) break;

    const int t = (int)(sg / a.sg_per_table);
    const int b0 = (int)(sg - (long long)t * a.sg_per_table) * a.bps;
    const int nb = min(a.bps, a.B - b0);
    const long long bag0 = (long long)t * a.B + b0;

    // offsets are clamped into [0, N] so that malformed input can never index
    // outside `indices`; lane j holds the offset of bag b0 + j
    int my_off = 0;
    if (lsg <= nb) my_off = (int)min(max(ld_idx<IDX>(a.offsets, bag0 + lsg), 0ll), (long long)N);
    const int P0 = __shfl(my_off, 0, LPR);
    const int P1 = __shfl(my_off, nb, LPR);

    const int c0 = lsg * CPL;
    const bool act = c0 < a.D;
    long long rows_t;
    const char* wbase;
    size_t rstride;
    if constexpr (SRC == 1) {
      rows_t = a.flat_rows;
      wbase = reinterpret_cast<const char*>(a.flat) + (size_t)c0 * Stor<DT>::kBytes;
      rstride = (size_t)a.D * Stor<DT>::kBytes;
    } else {
      rows_t = (long long)(a.row_off[t + 1] - a.row_off[t]);
      const int s = act ? c0 / a.Dsl : 0;
      const int cs = c0 - s * a.Dsl;
      wbase = reinterpret_cast<const char*>(a.tables[t].w[s]) + (size_t)cs * Stor<DT>::kBytes;
      rstride = (size_t)a.Dsl * Stor<DT>::kBytes;
    }
    HashMeta hm{};
    if constexpr (SRC == 2) hm = a.hmeta[t];
    const size_t ostride = (size_t)a.T * a.D;
    float* obase = a.out + (size_t)b0 * ostride + (size_t)t * a.D + c0;

    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

    int cur = 0;
    int cur_start = P0;
    int cur_end = __shfl(my_off, nb > 0 ? 1 : 0, LPR);
    int bad = 0;

    auto flush = [&](int L) {
      float* o = obase + (size_t)cur * ostride;
      if (act) {
        if (a.mean && L > 0) {
          const float fl = (float)L;
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] = __fdiv_rn(acc[c], fl);
        }
#pragma unroll
        for (int c = 0; c < CPL; c += 4) {
          f4 v = {acc[c], acc[c + 1], acc[c + 2], acc[c + 3]};
          __builtin_nontemporal_store(v, reinterpret_cast<f4*>(o + c));
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    };

    // SRC 0 / 1: the run's row indices are read LPR at a time, one per lane
    // of the subgroup, validated there, and handed out by lane shuffles, so
    // a row load waits on one round trip instead of an index load and then
    // its own. kNoRow marks an index outside the table (it adds nothing).
    // SRC 2 does the same with the ids: each lane probes the map for its own
    // lookup (home slot, then the probe sequence on a miss) and holds the
    // row, so the subgroup's probes run side by side. (Subgroups of fewer
    // than U lanes read each index in every lane.)
    constexpr uint32_t kNoRow = 0xffffffffu;
    constexpr bool kLaneIdx = LPR >= U;
    // row of lookup q (this lane's share of an index block), kNoRow if none
    auto row_of = [&](int q) -> uint32_t {
      uint32_t row = kNoRow;
      if (q < P1) {
        if constexpr (SRC == 2) {
          const long long id = reinterpret_cast<const long long*>(a.indices)[q];
          if (id != kEmpty) {  // an id without a row pools to nothing
            const long long s0 = hm.base + (uint32_t)(mix64((uint64_t)id) & hm.mask);
            const long long k0 = (long long)a.hkeys[s0];
            long long r = -1;
            if (k0 == id) {
              r = a.hvals[s0];
            } else if (k0 != kEmpty) {
              const long long slot = find_slot(hm, a.hkeys, id, false);
              if (slot >= 0) r = a.hvals[slot];
            }
            if (r >= 0 && r < rows_t) row = (uint32_t)r;
          }
        } else {
          long long r;
          if constexpr (SRC == 1) r = reinterpret_cast<const int32_t*>(a.indices)[q];
          else r = ld_idx<IDX>(a.indices, q);
          if (r >= 0 && r < rows_t) row = (uint32_t)r;
          else bad = 1;
        }
      }
      return row;
    };
    // The run's indices go by blocks of LPR lookups, one per lane. The next
    // block's indices are read while the current block's first rows are in
    // flight, so on long bags a row load never waits behind an index load
    // (SRC 2 probes a block when it reaches it: its probe chains would not
    // fit the registers twice).
    uint32_t myrow = kNoRow, nxrow = kNoRow;
    int blk_start = P0;  // first lookup of the block whose rows `myrow` holds
    if constexpr (kLaneIdx) myrow = row_of(P0 + lsg);
    for (int p = P0; p < P1; p += U) {
      if constexpr (kLaneIdx) {
        if (p >= blk_start + LPR) {  // uniform over the subgroup
          blk_start += LPR;
          if constexpr (SRC == 2) myrow = row_of(blk_start + lsg);
          else myrow = nxrow;
        }
      }
      // SRC 2: the U lookups' map probes are issued together -- ids, then the
      // home slots' keys, then the rows of the hits -- and only an id not in
      // its home slot walks the probe sequence
      long long hr[U];
      if constexpr (SRC == 2 && !kLaneIdx) {
        long long id[U];
        unsigned long long k0[U];
        long long s0[U];
#pragma unroll
        for (int k = 0; k < U; ++k)
          id[k] = p + k < P1 ? reinterpret_cast<const long long*>(a.indices)[p + k] : kEmpty;
#pragma unroll
        for (int k = 0; k < U; ++k) {
          s0[k] = hm.base + (uint32_t)(mix64((uint64_t)id[k]) & hm.mask);
          k0[k] = id[k] != kEmpty ? a.hkeys[s0[k]] : (unsigned long long)kEmpty;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
          hr[k] = -1;
          if ((long long)k0[k] == id[k] && id[k] != kEmpty) {
            hr[k] = a.hvals[s0[k]];
          } else if ((long long)k0[k] != kEmpty) {
            const long long slot = find_slot(hm, a.hkeys, id[k], false);
            if (slot >= 0) hr[k] = a.hvals[slot];
          }
        }
      }
      u4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        v[k] = u4{0u, 0u, 0u, 0u};
        if constexpr (SRC == 2 && !kLaneIdx) {
          const long long r = hr[k];
          if (p + k < P1 && r >= 0 && r < rows_t && act)
            v[k] = *reinterpret_cast<const u4*>(wbase + (size_t)r * rstride);
        } else if constexpr (!kLaneIdx) {
          if (p + k < P1) {
            long long r;
            if constexpr (SRC == 1) r = reinterpret_cast<const int32_t*>(a.indices)[p + k];
            else r = ld_idx<IDX>(a.indices, p + k);
            if (r >= 0 && r < rows_t) {
              if (act) v[k] = *reinterpret_cast<const u4*>(wbase + (size_t)r * rstride);
            } else {
              bad = 1;
            }
          }
        } else {
          // lookup p + k's row sits in lane (p + k - first of its block); U
          // divides LPR, so a group never straddles two blocks
          const uint32_t r = (uint32_t)__shfl((int)myrow, (p + k - blk_start) & (LPR - 1), LPR);
          if (p + k < P1 && r != kNoRow && act)
            v[k] = *reinterpret_cast<const u4*>(wbase + (size_t)r * rstride);
        }
      }
      if constexpr (kLaneIdx && SRC != 2) {
        if (p == blk_start && blk_start + LPR < P1) nxrow = row_of(blk_start + LPR + lsg);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (p + k < P1) {
          while (p + k >= cur_end && cur + 1 < nb) {
            flush(cur_end - cur_start);
            ++cur;
            cur_start = cur_end;
            cur_end = __shfl(my_off, cur + 1, LPR);
          }
          float f[CPL];
          widen16<DT>(v[k], f);
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] += f[c];
        }
      }
    }
    // the bag in progress, then any empty bags that close the run
    while (cur < nb) {
      flush(cur_end - cur_start);
      ++cur;
      cur_start = cur_end;
      cur_end = __shfl(my_off, min(cur + 1, nb), LPR);
    }
    if (bad) atomicOr(a.err, 1);
  }
}

#define FWD_LAUNCH(DT, IDX, LPR)                                                          \
  if (args.flat)                                                                       \
    hipLaunchKernelGGL((k_forward<DT, IDX, LPR, 1>), dim3(grid), dim3(256), 0, st, args); \
  else if (args.hmeta)                                                                 \
    hipLaunchKernelGGL((k_forward<DT, IDX, LPR, 2>), dim3(grid), dim3(256), 0, st, args); \
  else                                                                                 \
    hipLaunchKernelGGL((k_forward<DT, IDX, LPR, 0>), dim3(grid), dim3(256), 0, st, args); \
  break;

#define FWD_LPR_SWITCH(DT, IDX)                \
  switch (lpr) {                               \
    case 2: FWD_LAUNCH(DT, IDX, 2)             \
    case 4: FWD_LAUNCH(DT, IDX, 4)             \
    case 8: FWD_LAUNCH(DT, IDX, 8)             \
    case 16: FWD_LAUNCH(DT, IDX, 16)           \
    case 32: FWD_LAUNCH(DT, IDX, 32)           \
    default: FWD_LAUNCH(DT, IDX, 64)           \
  }

#define FWD_IDX_SWITCH(DT)                                   \
  if (itype == EMB_I32) {                                    \
    FWD_LPR_SWITCH(DT, int32_t)                              \
  } else {                                                   \
    FWD_LPR_SWITCH(DT, int64_t)                              \
  }

hipError_t launch_forward(const Geom& g, const DevCtx& dc, const void* indices, const void* offsets,
                          int itype, long long N, int B, int pool, float* out, int max_blocks,
                          hipStream_t st, const void* flat, long long flat_rows, const HashView* hash) {
  if (B == 0 || g.T == 0) return hipSuccess;
  const int cpl = 16 / (g.dtype == EMB_F32 ? 4 : 2);
  int lpr = next_pow2((g.D + cpl - 1) / cpl);
  if (lpr < 2) lpr = 2;
  // about 16 lookups per subgroup run, at most lpr-1 bags (one offset per lane)
  const double avg = (double)N / ((double)g.T * (double)B);
  int bps = avg > 0 ? (int)(16.0 / avg + 0.5) : lpr - 1;
  if (bps < 1) bps = 1;
  if (bps > lpr - 1) bps = lpr - 1;
  if (bps > B) bps = B;
  FwdArgs args;
  args.indices = indices;
  args.offsets = offsets;
  args.tables = dc.tables;
  args.row_off = dc.row_off;
  args.out = out;
  args.err = dc.err_flag;
  args.N = N;
  args.T = g.T;
  args.B = B;
  args.D = g.D;
  args.Dsl = g.Dsl;
  args.bps = bps;
  args.sg_per_table = ceil_div(B, bps);
  args.total_sg = (long long)g.T * args.sg_per_table;
  const int sgw = 256 / lpr;
  args.nblk = (int)((args.total_sg + sgw - 1) / sgw);
  args.mean = pool == EMB_POOL_MEAN;
  args.flat = flat;
  args.flat_rows = flat_rows;
  args.hmeta = hash ? hash->meta : nullptr;
  args.hkeys = hash ? hash->keys : nullptr;
  args.hvals = hash ? hash->vals : nullptr;
  const int grid = max_blocks > 0 && max_blocks < args.nblk ? max_blocks : round_up8(args.nblk);
  switch (g.dtype) {
    case EMB_F32:
      FWD_IDX_SWITCH(EMB_F32)
      break;
    case EMB_BF16:
      FWD_IDX_SWITCH(EMB_BF16)
      break;
    default:
      FWD_IDX_SWITCH(EMB_F16)
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// unique rows -> compact buffer
// ---------------------------------------------------------------------------

// One subgroup of LPR lanes per unique key u < U: its logical row (all column
// slices) is copied, in the storage type, to rows[u]; the invalid-index
// sentinel key gets a zero row (such lookups pool to nothing, as in the
// direct forward).
template <int DT, int LPR>
__global__ __launch_bounds__(256) void k_gather_unique(const DevTable* __restrict__ tables,
                                                       const uint32_t* __restrict__ row_off,
                                                       const uint32_t* __restrict__ ukeys,
                                                       const int32_t* __restrict__ num_unique, int cap,
                                                       int T, int D, int Dsl, uint32_t total_rows,
                                                       void* __restrict__ rows) {
  extern __shared__ uint32_t s_ro[];
  for (int i = threadIdx.x; i <= T; i += 256) s_ro[i] = row_off[i];
  __syncthreads();
  constexpr int CPL = 16 / Stor<DT>::kBytes;
  constexpr int SGW = 256 / LPR;
  const int lsg = threadIdx.x & (LPR - 1);
  const int c0 = lsg * CPL;
  if (c0 >= D) return;
  const int U = min(max(*num_unique, 0), cap);
  const size_t rbytes = (size_t)D * Stor<DT>::kBytes;
  for (long long u = (long long)blockIdx.x * SGW + threadIdx.x / LPR; u < U; u += (long long)gridDim.x * SGW) {
    const uint32_t key = ukeys[u];
    u4 v = {0u, 0u, 0u, 0u};
    if (key < total_rows) {
      const int t = table_of(s_ro, T, key);
      const int s = c0 / Dsl;
      const size_t e = (size_t)(key - s_ro[t]) * Dsl + (c0 - s * Dsl);
      v = *reinterpret_cast<const u4*>(reinterpret_cast<const char*>(tables[t].w[s]) + e * Stor<DT>::kBytes);
    }
    *reinterpret_cast<u4*>(reinterpret_cast<char*>(rows) + (size_t)u * rbytes + (size_t)c0 * Stor<DT>::kBytes) = v;
  }
}

hipError_t launch_gather_unique(const Geom& g, const DevCtx& dc, const uint32_t* ukeys,
                                const int32_t* num_unique, int cap, void* rows, hipStream_t st) {
  if (cap <= 0) return hipSuccess;
  const int cpl = 16 / (g.dtype == EMB_F32 ? 4 : 2);
  int lpr = next_pow2((g.D + cpl - 1) / cpl);
  if (lpr < 2) lpr = 2;
  const int sgw = 256 / lpr;
  const long long want = ((long long)cap + sgw - 1) / sgw;
  const int grid = (int)(want < 16384 ? want : 16384);
  const size_t smem = (size_t)(g.T + 1) * 4;
#define GU(DT, P)                                                                                       \
  hipLaunchKernelGGL((k_gather_unique<DT, P>), dim3(grid), dim3(256), smem, st, dc.tables, dc.row_off, \
                     ukeys, num_unique, cap, g.T, g.D, g.Dsl, g.total_rows, rows);                      \
  break;
#define GU_LPR(DT)             \
  switch (lpr) {               \
    case 2: GU(DT, 2)          \
    case 4: GU(DT, 4)          \
    case 8: GU(DT, 8)          \
    case 16: GU(DT, 16)        \
    case 32: GU(DT, 32)        \
    default: GU(DT, 64)        \
  }
  switch (g.dtype) {
    case EMB_F32:
      GU_LPR(EMB_F32)
      break;
    case EMB_BF16:
      GU_LPR(EMB_BF16)
      break;
    default:
      GU_LPR(EMB_F16)
      break;
  }
#undef GU_LPR
#undef GU
  return hipGetLastError();
}

}  // namespace emb
