// Routing the step's unique keys to their owner shards (EMBark, RecSys'24
// article: embedding clusters that send each distinct key, and its reduced
// gradient, once; shards from its 3D sharding). For one GPU's share this is
// the layout step before an all-to-all:
//   dest    unique key u -> word (dest(u) << 32 | u); the owner comes from the
//           table's rule (whole table / cyclic rows / row blocks); lookups past
//           the unique count and the invalid-index sentinel get dest = S
//   sort    the radix-sort pass kernels order the words by dest, stably, so
//           keys stay ascending inside a destination
//   place   send_keys[i] = key of the i-th word, slot_of_unique[u] = i
//   offsets send_offsets[s] = first i whose dest >= s (binary search)
// The reduced gradients of RB are then written by the segmented reduce
// straight into their slots (k_reduce.hip, slot map).
#include "emb_device.h"

namespace emb {

struct PackArgs {
  const uint32_t* ukeys;
  const int32_t* num_unique;
  const uint32_t* row_off;
  const int2* rules;  // [T] {kind, shard}
  uint64_t* words;
  int N, T, S;
  uint32_t total_rows;
};

__global__ __launch_bounds__(256) void k_pack_dest(PackArgs a) {
  extern __shared__ uint32_t s_ro[];
  for (int i = threadIdx.x; i <= a.T; i += 256) s_ro[i] = a.row_off[i];
  __syncthreads();
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= a.N) return;
  const int U = min(max(*a.num_unique, 0), a.N);
  uint32_t dest = (uint32_t)a.S;
  if (u < U) {
    const uint32_t key = a.ukeys[u];
    if (key < a.total_rows) {
      const int t = table_of(s_ro, a.T, key);
      const uint32_t r = key - s_ro[t];
      const uint32_t rows = s_ro[t + 1] - s_ro[t];
      const int2 rule = a.rules[t];
      if (rule.x == EMB_SHARD_TABLE) {
        dest = (uint32_t)rule.y;
      } else if (rule.x == EMB_SHARD_ROW_CYCLIC) {
        dest = (uint32_t)(((uint64_t)r + (uint32_t)rule.y) % (uint32_t)a.S);
      } else {
        const uint32_t block = (uint32_t)(((uint64_t)rows + a.S - 1) / (uint32_t)a.S);
        dest = r / block;
      }
    }
  }
  a.words[u] = ((uint64_t)dest << 32) | (uint32_t)u;
}

__global__ __launch_bounds__(256) void k_pack_place(const uint64_t* __restrict__ sorted,
                                                    const uint32_t* __restrict__ ukeys,
                                                    const int32_t* __restrict__ num_unique, int N, int S,
                                                    uint32_t* __restrict__ send_keys,
                                                    int32_t* __restrict__ slot) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const uint64_t w = sorted[i];
  const uint32_t d = (uint32_t)(w >> 32);
  const uint32_t u = (uint32_t)w;
  if (u >= (uint32_t)N) return;
  if (d < (uint32_t)S) {
    send_keys[i] = ukeys[u];
    slot[u] = i;
  } else if ((int)u < min(max(*num_unique, 0), N)) {
    slot[u] = -1;  // the invalid-index sentinel: sent nowhere
  }
}

__global__ __launch_bounds__(256) void k_pack_offsets(const uint64_t* __restrict__ sorted, int N, int S,
                                                      int32_t* __restrict__ send_offsets) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s > S) return;
  int lo = 0, hi = N;  // first i in [0, N] with dest(i) >= s
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((uint32_t)(sorted[mid] >> 32) < (uint32_t)s) lo = mid + 1;
    else hi = mid;
  }
  send_offsets[s] = lo;
}

hipError_t launch_pack_dest(const Geom& g, const DevCtx& dc, const int2* rules, int S, int N,
                            const uint32_t* ukeys, const int32_t* num_unique, uint64_t* words,
                            hipStream_t st) {
  PackArgs a;
  a.ukeys = ukeys;
  a.num_unique = num_unique;
  a.row_off = dc.row_off;
  a.rules = rules;
  a.words = words;
  a.N = N;
  a.T = g.T;
  a.S = S;
  a.total_rows = g.total_rows;
  const int grid = ceil_div(N, 256);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_dest, dim3(grid), dim3(256), (size_t)(g.T + 1) * 4, st, a);
  return hipGetLastError();
}

hipError_t launch_pack_place(const uint64_t* sorted, const uint32_t* ukeys, const int32_t* num_unique,
                             int N, int S, uint32_t* send_keys, int32_t* slot, hipStream_t st) {
  const int grid = ceil_div(N, 256);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_place, dim3(grid), dim3(256), 0, st, sorted, ukeys, num_unique, N, S,
                     send_keys, slot);
  return hipGetLastError();
}

hipError_t launch_pack_offsets(const uint64_t* sorted, int N, int S, int32_t* send_offsets,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_pack_offsets, dim3(ceil_div(S + 1, 256)), dim3(256), 0, st, sorted, N, S,
                     send_offsets);
  return hipGetLastError();
}

}  // namespace emb
