// Synthetic table contents (set-up, outside a training step).
//
// Element (t, r, c) of a table with logical width D becomes
//   v = (splitmix64(seed ^ (t << 40) ^ (r*D + c)) >> 40) - 2^23   (integer in [-2^23, 2^23))
//   w = fp32(v) * fp32(0.1f * 2^-24)                               (one rounded multiply)
// i.e. U(-0.05, 0.05), then rounded to the storage type (RNE); a table with an
// fp32 master holds w itself there and its RNE cast in the storage. SplitMix64 is
// the generator of Steele, Lea & Flood ("Fast splittable pseudorandom number
// generators", OOPSLA 2014): add the golden gamma, then the variant-13 mixer.
// The Adagrad accumulator (if any) starts at 0.
#include "emb_device.h"

namespace emb {

__device__ __forceinline__ uint64_t splitmix64_dev(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float init_value(uint64_t seed, int t, uint64_t lin) {
  const uint64_t h = splitmix64_dev(seed ^ ((uint64_t)t << 40) ^ lin);
  const int32_t v = (int32_t)(h >> 40) - (1 << 23);
  const float scale = 0.1f * 0x1p-24f;
  return __fmul_rn((float)v, scale);
}

template <int DT>
__global__ __launch_bounds__(256) void k_init_slice(void* w, float* state, float* master,
                                                    int64_t rows, int D, int Dsl, int s, int t,
                                                    uint64_t seed) {
  const int qpr = Dsl / 4;  // quads per slice row
  const int64_t nq = rows * (int64_t)qpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride) {
    const int64_t r = q / qpr;
    const int cq = (int)(q - r * qpr) * 4;
    const uint64_t lin = (uint64_t)r * (uint64_t)D + (uint64_t)(s * Dsl + cq);
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = init_value(seed, t, lin + k);
    char* p = reinterpret_cast<char*>(w) + (size_t)(r * Dsl + cq) * Stor<DT>::kBytes;
    store4<DT>(p, v);
    if (master) {
      f4 m = {v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f4*>(master + r * Dsl + cq) = m;
    }
    if (state) {
      f4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f4*>(state + r * Dsl + cq) = z;
    }
  }
}

hipError_t launch_init_slice(const Geom& g, const DevCtx& dc, int t, int s, int64_t rows, void* w,
                             float* state, float* master, uint64_t seed, hipStream_t st) {
  (void)dc;
  const int64_t nq = rows * (g.Dsl / 4);
  const int64_t want = (nq + 255) / 256;
  const int blocks = (int)(want < 32768 ? (want > 0 ? want : 1) : 32768);
  switch (g.dtype) {
    case EMB_F32:
      hipLaunchKernelGGL(k_init_slice<EMB_F32>, dim3(blocks), dim3(256), 0, st, w, state, master, rows, g.D,
                         g.Dsl, s, t, seed);
      break;
    case EMB_BF16:
      hipLaunchKernelGGL(k_init_slice<EMB_BF16>, dim3(blocks), dim3(256), 0, st, w, state, master, rows,
                         g.D, g.Dsl, s, t, seed);
      break;
    default:
      hipLaunchKernelGGL(k_init_slice<EMB_F16>, dim3(blocks), dim3(256), 0, st, w, state, master, rows,
                         g.D, g.Dsl, s, t, seed);
      break;
  }
  return hipGetLastError();
}

}  // namespace emb
