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
// the storage type with round-to-nearest-even. Rows no lookup touched are
// never read or written.
//
// Work split. Segments are cut into chunks (at segment starts and every
// kChunk sorted positions). One subgroup of LPR lanes (4 fp32 columns per
// lane, so a dY row is one coalesced access) reduces one chunk, keeping 8 dY
// rows in flight; a chunk that is a whole segment applies the optimizer
// right there with the weight (and state) row prefetched before the dY loop,
// so the reduced gradient never leaves VGPRs. A segment longer than a tile
// leaves one partial per tile it touches (at most two partial slots per
// tile), and the combine kernel adds them in tile order -- a fixed order, so
// results are bit-reproducible run to run -- with the whole block, then
// applies the update. No atomics touch gradients or weights.
#include "emb_device.h"

namespace emb {

struct RedArgs {
  const int32_t* sorted_bag;
  const float* inv_len;  // null for sum pooling
  const float* dY;
  const uint32_t* ukeys;
  const int32_t* seg_off;
  const int32_t* chunk_off;
  const int32_t* chunk_seg;
  const int32_t* num_chunks;
  const int32_t* num_unique;
  const int32_t* tile_last_seg;
  float* partial;
  float* grad;  // reduced gradient out (mode 0) or in (apply)
  const DevTable* tables;
  const uint32_t* row_off;
  int T, B, D, Dsl;
  uint32_t total_rows;
  int N;
  int ntiles;
  float lr, eps;
};

__device__ __forceinline__ int table_of(const uint32_t* s_ro, int T, uint32_t key) {
  int lo = 0, hi = T;  // s_ro[lo] <= key < s_ro[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_ro[mid] <= key) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <int DT>
__device__ __forceinline__ void row_ptrs(const RedArgs& a, int t, uint32_t r, int c0, char** wp,
                                         float** gp) {
  const int s = c0 / a.Dsl;
  const int cs = c0 - s * a.Dsl;
  const size_t e = (size_t)r * a.Dsl + cs;
  *wp = reinterpret_cast<char*>(a.tables[t].w[s]) + e * Stor<DT>::kBytes;
  float* g = a.tables[t].g[s];
  *gp = g ? g + e : nullptr;
}

// mode 1 = SGD, 2 = Adagrad
template <int DT, int MODE>
__device__ __forceinline__ void row_update(char* wp, float* gp, const float* wv, const float* Gv,
                                           const float* g, float lr, float eps) {
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
  store4<DT>(wp, nw);
}

template <int DT, int LPR, int MODE>
__global__ __launch_bounds__(256) void k_chunks(RedArgs a) {
  extern __shared__ uint32_t s_ro[];
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  __syncthreads();
  constexpr int U = 8;
  constexpr int SGW = 256 / LPR;
  const int lsg = threadIdx.x & (LPR - 1);
  const int c0 = lsg * 4;
  const bool act = c0 < a.D;
  const size_t dys = (size_t)a.T * a.D;
  const long long nsg = (long long)gridDim.x * SGW;
  const int nch = min(*a.num_chunks, a.N + a.ntiles);
  for (long long q = (long long)blockIdx.x * SGW + threadIdx.x / LPR; q < nch; q += nsg) {
    // every index below is clamped into its buffer: a wrong count or offset
    // can give a wrong result, never an access outside the workspace
    const int cb = max(a.chunk_off[q], 0);
    const int ce = min(a.chunk_off[q + 1], a.N);
    const int u = a.chunk_seg[q];
    if (u < 0 || u >= a.N) continue;
    const int so = a.seg_off[u];
    const int eo = a.seg_off[u + 1];
    const uint32_t key = a.ukeys[u];
    if (key >= a.total_rows) continue;  // lookups with out-of-range indices
    const int t = table_of(s_ro, a.T, key);
    const uint32_t r = key - s_ro[t];
    const bool whole = cb == so && ce == eo;

    char* wp = nullptr;
    float* gp = nullptr;
    float wv[4] = {0.f, 0.f, 0.f, 0.f}, Gv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE != 0) {
      if (whole && act) {
        row_ptrs<DT>(a, t, r, c0, &wp, &gp);
        load4<DT>(wp, wv);
        if constexpr (MODE == 2) load4<EMB_F32>(gp, Gv);
      }
    }

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const float* dyt = a.dY + (size_t)t * a.D + c0;
    const int bagt = t * a.B;
    for (int i = cb; i < ce; i += U) {
      int bg[U];
#pragma unroll
      for (int k = 0; k < U; ++k) bg[k] = i + k < ce ? a.sorted_bag[i + k] : -1;
      f4 v[U];
      float sc[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        v[k] = f4{0.f, 0.f, 0.f, 0.f};
        sc[k] = 1.f;
        if (bg[k] >= 0) {
          const unsigned b = (unsigned)(bg[k] - bagt);
          if (b < (unsigned)a.B) {
            if (act) v[k] = *reinterpret_cast<const f4*>(dyt + (size_t)b * dys);
            if (a.inv_len) sc[k] = a.inv_len[bg[k]];
          }
        }
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (bg[k] >= 0) {
          if (a.inv_len) {
            acc[0] += sc[k] * v[k].x;
            acc[1] += sc[k] * v[k].y;
            acc[2] += sc[k] * v[k].z;
            acc[3] += sc[k] * v[k].w;
          } else {
            acc[0] += v[k].x;
            acc[1] += v[k].y;
            acc[2] += v[k].z;
            acc[3] += v[k].w;
          }
        }
      }
    }

    if (!act) continue;
    if (whole) {
      if constexpr (MODE == 0) {
        f4 o = {acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f4*>(a.grad + (size_t)u * a.D + c0) = o;
      } else {
        row_update<DT, MODE>(wp, gp, wv, Gv, acc, a.lr, a.eps);
      }
    } else {
      const int j = cb / kChunk;
      const int slot = 2 * j + (cb == j * kChunk ? 0 : 1);
      f4 o = {acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f4*>(a.partial + (size_t)slot * a.D + c0) = o;
    }
  }
}

// Long segments: the block finds, among 256 tiles, the segments that start in
// a tile and run past its end (one per tile at most: the tile's last
// segment), then reduces each one's partials cooperatively.
template <int DT, int LPR, int MODE>
__global__ __launch_bounds__(256) void k_combine(RedArgs a) {
  constexpr int SGW = 256 / LPR;
  extern __shared__ uint32_t smem[];
  uint32_t* s_ro = smem;
  const int ro_words = (a.T + 1 + 3) & ~3;
  float* s_part = reinterpret_cast<float*>(smem + ro_words);  // [SGW][4*LPR]
  int* s_list = reinterpret_cast<int*>(s_part + SGW * 4 * LPR);  // [256]
  __shared__ int s_n;
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  const int sg = threadIdx.x / LPR;
  const int lsg = threadIdx.x & (LPR - 1);
  const int c0 = lsg * 4;
  const bool act = c0 < a.D;
  for (long long tb = (long long)blockIdx.x * 256; tb < a.ntiles; tb += (long long)gridDim.x * 256) {
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    const long long j = tb + threadIdx.x;
    if (j < a.ntiles && (unsigned)a.tile_last_seg[j] < (unsigned)a.N) {
      const int u = a.tile_last_seg[j];
      const long long so = a.seg_off[u];
      const long long eo = a.seg_off[u + 1];
      if (so >= j * kChunk && eo > (j + 1) * kChunk && a.ukeys[u] < a.total_rows) {
        const int p = atomicAdd(&s_n, 1);
        s_list[p] = u;
      }
    }
    __syncthreads();
    const int n = s_n;
    for (int e = 0; e < n; ++e) {
      const int u = s_list[e];
      const int so = a.seg_off[u];
      const int eo = a.seg_off[u + 1];
      const int j0 = so / kChunk;
      const int np = (eo - 1) / kChunk - j0 + 1;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      constexpr int U = 4;
      for (int k0 = sg; k0 < np; k0 += SGW * U) {
        f4 v[U];
#pragma unroll
        for (int m = 0; m < U; ++m) {
          const int k = k0 + m * SGW;
          v[m] = f4{0.f, 0.f, 0.f, 0.f};
          if (k < np && act) {
            const int slot = k == 0 ? (so == j0 * kChunk ? 2 * j0 : 2 * j0 + 1) : 2 * (j0 + k);
            v[m] = *reinterpret_cast<const f4*>(a.partial + (size_t)slot * a.D + c0);
          }
        }
#pragma unroll
        for (int m = 0; m < U; ++m) {
          acc[0] += v[m].x;
          acc[1] += v[m].y;
          acc[2] += v[m].z;
          acc[3] += v[m].w;
        }
      }
      if (act) {
        float* sp = s_part + (size_t)sg * 4 * LPR + c0;
        sp[0] = acc[0];
        sp[1] = acc[1];
        sp[2] = acc[2];
        sp[3] = acc[3];
      }
      __syncthreads();
      if (sg == 0 && act) {
        float g[4] = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < SGW; ++k) {
          const float* sp = s_part + (size_t)k * 4 * LPR + c0;
          g[0] += sp[0];
          g[1] += sp[1];
          g[2] += sp[2];
          g[3] += sp[3];
        }
        const uint32_t key = a.ukeys[u];
        if constexpr (MODE == 0) {
          f4 o = {g[0], g[1], g[2], g[3]};
          *reinterpret_cast<f4*>(a.grad + (size_t)u * a.D + c0) = o;
        } else {
          const int t = table_of(s_ro, a.T, key);
          char* wp;
          float* gp;
          row_ptrs<DT>(a, t, key - s_ro[t], c0, &wp, &gp);
          float wv[4], Gv[4] = {0.f, 0.f, 0.f, 0.f};
          load4<DT>(wp, wv);
          if constexpr (MODE == 2) load4<EMB_F32>(gp, Gv);
          row_update<DT, MODE>(wp, gp, wv, Gv, g, a.lr, a.eps);
        }
      }
      __syncthreads();
    }
    __syncthreads();
  }
}

// Update from a materialised reduced gradient (grad[u] for u < U).
template <int DT, int LPR, int MODE>
__global__ __launch_bounds__(256) void k_apply(RedArgs a) {
  extern __shared__ uint32_t s_ro[];
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  __syncthreads();
  constexpr int SGW = 256 / LPR;
  const int lsg = threadIdx.x & (LPR - 1);
  const int c0 = lsg * 4;
  if (c0 >= a.D) return;
  const int U = min(*a.num_unique, a.N);
  for (long long u = (long long)blockIdx.x * SGW + threadIdx.x / LPR; u < U;
       u += (long long)gridDim.x * SGW) {
    const uint32_t key = a.ukeys[u];
    if (key >= a.total_rows) continue;
    const int t = table_of(s_ro, a.T, key);
    char* wp;
    float* gp;
    row_ptrs<DT>(a, t, key - s_ro[t], c0, &wp, &gp);
    float wv[4], Gv[4] = {0.f, 0.f, 0.f, 0.f}, g[4];
    load4<DT>(wp, wv);
    if constexpr (MODE == 2) load4<EMB_F32>(gp, Gv);
    load4<EMB_F32>(a.grad + (size_t)u * a.D + c0, g);
    row_update<DT, MODE>(wp, gp, wv, Gv, g, a.lr, a.eps);
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
  a.chunk_off = reinterpret_cast<const int32_t*>(ws + L.chunk_off);
  a.chunk_seg = reinterpret_cast<const int32_t*>(ws + L.chunk_seg);
  a.num_chunks = reinterpret_cast<const int32_t*>(ws + L.scalars);
  a.num_unique = nullptr;
  a.tile_last_seg = reinterpret_cast<const int32_t*>(ws + L.tile_last_seg);
  a.partial = const_cast<float*>(reinterpret_cast<const float*>(ws + L.partial));
  a.grad = nullptr;
  a.tables = dc.tables;
  a.row_off = dc.row_off;
  a.T = g.T;
  a.B = 0;
  a.D = g.D;
  a.Dsl = g.Dsl;
  a.total_rows = g.total_rows;
  a.N = N;
  a.ntiles = L.ntiles;
  a.lr = lr;
  a.eps = eps;
  return a;
}

static int lpr_b(const Geom& g) {
  int l = next_pow2((g.D + 3) / 4);
  return l < 2 ? 2 : l;
}

#define RED_KERNEL_SWITCH(KERNEL, DT, MODE, GRID, SMEM)                                 \
  switch (lpr) {                                                                        \
    case 2: hipLaunchKernelGGL((KERNEL<DT, 2, MODE>), GRID, dim3(256), SMEM, st, a); break;   \
    case 4: hipLaunchKernelGGL((KERNEL<DT, 4, MODE>), GRID, dim3(256), SMEM, st, a); break;   \
    case 8: hipLaunchKernelGGL((KERNEL<DT, 8, MODE>), GRID, dim3(256), SMEM, st, a); break;   \
    case 16: hipLaunchKernelGGL((KERNEL<DT, 16, MODE>), GRID, dim3(256), SMEM, st, a); break; \
    case 32: hipLaunchKernelGGL((KERNEL<DT, 32, MODE>), GRID, dim3(256), SMEM, st, a); break; \
    default: hipLaunchKernelGGL((KERNEL<DT, 64, MODE>), GRID, dim3(256), SMEM, st, a); break; \
  }

#define RED_MODE_SWITCH(KERNEL, DT, GRID, SMEM)             \
  if (mode == 0) {                                          \
    RED_KERNEL_SWITCH(KERNEL, DT, 0, GRID, SMEM)            \
  } else if (mode == 1) {                                   \
    RED_KERNEL_SWITCH(KERNEL, DT, 1, GRID, SMEM)            \
  } else {                                                  \
    RED_KERNEL_SWITCH(KERNEL, DT, 2, GRID, SMEM)            \
  }

#define RED_DISPATCH(KERNEL, GRID, SMEM)                    \
  switch (g.dtype) {                                        \
    case EMB_F32: RED_MODE_SWITCH(KERNEL, EMB_F32, GRID, SMEM) break;   \
    case EMB_BF16: RED_MODE_SWITCH(KERNEL, EMB_BF16, GRID, SMEM) break; \
    default: RED_MODE_SWITCH(KERNEL, EMB_F16, GRID, SMEM) break;        \
  }

hipError_t launch_reduce(const Geom& g, const DevCtx& dc, int mode, int N, int B, int pool,
                         const float* dY, const WsLayout& L, const char* ws,
                         const uint32_t* unique_keys, const int32_t* num_unique, float* grad_out,
                         float lr, float eps, hipStream_t st) {
  RedArgs a = make_args(g, dc, N, L, ws, unique_keys, lr, eps);
  a.B = B;
  a.dY = dY;
  a.inv_len = pool == EMB_POOL_MEAN ? reinterpret_cast<const float*>(ws + L.inv_len) : nullptr;
  a.num_unique = num_unique;
  a.grad = grad_out;
  const int lpr = lpr_b(g);
  const int sgw = 256 / lpr;
  // chunks <= N + ntiles; the loop is grid-strided over the device count
  const long long upper = (long long)N + L.ntiles;
  long long want = (upper + sgw - 1) / sgw;
  const int grid = (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
  const size_t smem = (size_t)(g.T + 1) * 4;
  RED_DISPATCH(k_chunks, dim3(grid), smem)
  return hipGetLastError();
}

hipError_t launch_combine(const Geom& g, const DevCtx& dc, int mode, int N, const WsLayout& L,
                          const char* ws, const uint32_t* unique_keys, float* grad_out, float lr,
                          float eps, hipStream_t st) {
  RedArgs a = make_args(g, dc, N, L, ws, unique_keys, lr, eps);
  a.grad = grad_out;
  const int lpr = lpr_b(g);
  const int sgw = 256 / lpr;
  const int want = ceil_div(L.ntiles, 256);
  const int grid = want < 4096 ? (want > 0 ? want : 1) : 4096;
  const size_t smem = (size_t)((g.T + 1 + 3) & ~3) * 4 + (size_t)sgw * 4 * lpr * 4 + 256 * 4;
  RED_DISPATCH(k_combine, dim3(grid), smem)
  return hipGetLastError();
}

hipError_t launch_apply(const Geom& g, const DevCtx& dc, int opt, int N,
                        const uint32_t* unique_keys, const int32_t* num_unique,
                        const float* grad_in, float lr, float eps, hipStream_t st) {
  RedArgs a;
  a.sorted_bag = nullptr;
  a.inv_len = nullptr;
  a.dY = nullptr;
  a.ukeys = unique_keys;
  a.seg_off = a.chunk_off = a.chunk_seg = a.num_chunks = a.tile_last_seg = nullptr;
  a.num_unique = num_unique;
  a.partial = nullptr;
  a.grad = const_cast<float*>(grad_in);
  a.tables = dc.tables;
  a.row_off = dc.row_off;
  a.T = g.T;
  a.B = 0;
  a.D = g.D;
  a.Dsl = g.Dsl;
  a.total_rows = g.total_rows;
  a.N = N;
  a.ntiles = 0;
  a.lr = lr;
  a.eps = eps;
  const int lpr = lpr_b(g);
  const int sgw = 256 / lpr;
  const long long want = ((long long)N + sgw - 1) / sgw;
  const int grid = (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
  const size_t smem = (size_t)(g.T + 1) * 4;
  const int mode = opt;
  if (mode == 1) {
    switch (g.dtype) {
      case EMB_F32: RED_KERNEL_SWITCH(k_apply, EMB_F32, 1, dim3(grid), smem) break;
      case EMB_BF16: RED_KERNEL_SWITCH(k_apply, EMB_BF16, 1, dim3(grid), smem) break;
      default: RED_KERNEL_SWITCH(k_apply, EMB_F16, 1, dim3(grid), smem) break;
    }
  } else {
    switch (g.dtype) {
      case EMB_F32: RED_KERNEL_SWITCH(k_apply, EMB_F32, 2, dim3(grid), smem) break;
      case EMB_BF16: RED_KERNEL_SWITCH(k_apply, EMB_BF16, 2, dim3(grid), smem) break;
      default: RED_KERNEL_SWITCH(k_apply, EMB_F16, 2, dim3(grid), smem) break;
    }
  }
  return hipGetLastError();
}

}  // namespace emb
