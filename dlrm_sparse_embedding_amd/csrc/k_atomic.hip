// Evidence variant of the backward reduction: per-lookup fp32 atomics
// instead of sorted segments.
//
// The reduced gradient of unique key u is the same sum as in the sorted path,
// sum over lookups i with inverse[i] == u of scale_i * dY[b(i)][t(i)*D ...]
// (EMBark's reduction-based compression, applied locally), but accumulated by
// hardware fp32 atomic adds (global_atomic_add_f32) into reduced_grad[u]:
// one subgroup per bag loads the bag's dY row once and adds it into the row of
// every lookup of the bag. The summation order is whatever order the atomics
// land in, so results are correct up to fp32 rounding but not bit-reproducible.
// It exists to measure atomics against the sorted-segment reduction.
#include "emb_device.h"

namespace emb {

__global__ __launch_bounds__(256) void k_zero_rows(float* __restrict__ grad,
                                                   const int32_t* __restrict__ num_unique, int D,
                                                   int N) {
  const long long n = (long long)min(*num_unique, N) * D;  // D % 4 == 0
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  for (long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4; i < n;
       i += (long long)gridDim.x * 256 * 4)
    *reinterpret_cast<f4*>(grad + i) = z;
}

struct AtomArgs {
  const void* offsets;
  const float* dY;
  const int32_t* inverse;
  const int32_t* num_unique;
  float* grad;
  long long N;
  int T, B, D;
};

template <typename IDX, int LPR, bool MEAN>
__global__ __launch_bounds__(256) void k_atomic_scatter(AtomArgs a) {
  constexpr int SGW = 256 / LPR;
  const int c0 = (int)blockIdx.y * 4 * LPR + (threadIdx.x & (LPR - 1)) * 4;  // column block: blockIdx.y
  const bool act = c0 < a.D;
  const int U = min(*a.num_unique, (int)a.N);
  const long long bags = (long long)a.T * a.B;
  for (long long bag = (long long)blockIdx.x * SGW + threadIdx.x / LPR; bag < bags;
       bag += (long long)gridDim.x * SGW) {
    const long long s = min(max(ld_idx<IDX>(a.offsets, bag), 0ll), a.N);
    const long long e = min(max(ld_idx<IDX>(a.offsets, bag + 1), s), a.N);
    if (e == s) continue;
    const int t = (int)(bag / a.B);
    const long long b = bag - (long long)t * a.B;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (act) v = *reinterpret_cast<const f4*>(a.dY + (size_t)b * a.T * a.D + (size_t)t * a.D + c0);
    if constexpr (MEAN) v *= __fdiv_rn(1.0f, (float)(e - s));
    for (long long i = s; i < e; ++i) {
      const int u = a.inverse[i];
      if (act && (unsigned)u < (unsigned)U) {
        float* g = a.grad + (size_t)u * a.D + c0;
        unsafeAtomicAdd(g + 0, v.x);
        unsafeAtomicAdd(g + 1, v.y);
        unsafeAtomicAdd(g + 2, v.z);
        unsafeAtomicAdd(g + 3, v.w);
      }
    }
  }
}

hipError_t launch_atomic_reduce(const Geom& g, const void* offsets, int itype, long long N, int B,
                                int pool, const float* dY, const int32_t* inverse,
                                const int32_t* num_unique, float* grad, hipStream_t st) {
  const int zgrid = (int)std::min<long long>(((long long)N * g.D / 4 + 255) / 256 + 1, 8192);
  hipLaunchKernelGGL(k_zero_rows, dim3(zgrid), dim3(256), 0, st, grad, num_unique, g.D, (int)N);
  AtomArgs a{offsets, dY, inverse, num_unique, grad, N, g.T, B, g.D};
  int lpr = next_pow2((g.D + 3) / 4);
  if (lpr < 2) lpr = 2;
  if (lpr > 64) lpr = 64;  // wider rows take col_blocks() blocks along y
  const int sgw = 256 / lpr;
  const long long bags = (long long)g.T * B;
  const int grid = (int)std::min<long long>((bags + sgw - 1) / sgw, 16384);
  const bool mean = pool == EMB_POOL_MEAN;
#define L_AT(IDX, P)                                                                           \
  if (mean) hipLaunchKernelGGL((k_atomic_scatter<IDX, P, true>), dim3(grid, col_blocks(g.D, P)), dim3(256), 0, st, a); \
  else hipLaunchKernelGGL((k_atomic_scatter<IDX, P, false>), dim3(grid, col_blocks(g.D, P)), dim3(256), 0, st, a);
#define L_AT_LPR(IDX)                   \
  switch (lpr) {                        \
    case 2: L_AT(IDX, 2) break;         \
    case 4: L_AT(IDX, 4) break;         \
    case 8: L_AT(IDX, 8) break;         \
    case 16: L_AT(IDX, 16) break;       \
    case 32: L_AT(IDX, 32) break;       \
    default: L_AT(IDX, 64) break;       \
  }
  if (grid > 0) {
    if (itype == EMB_I32) {
      L_AT_LPR(int32_t)
    } else {
      L_AT_LPR(int64_t)
    }
  }
#undef L_AT_LPR
#undef L_AT
  return hipGetLastError();
}

}  // namespace emb
