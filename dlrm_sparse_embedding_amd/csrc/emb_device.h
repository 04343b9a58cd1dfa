// Device helpers for the gfx950 kernels: storage conversions, vector
// loads/stores, wave-level primitives, XCD-aware block mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "emb_internal.h"

namespace emb {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// ---- storage types ------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return ((b >> 16) | 0x40u) & 0xffffu;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// binary16 -> fp32, exact, written on the bit fields so that no hardware
// denormal mode can flush a subnormal half.
__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  const uint32_t sign = (h16 & 0x8000u) << 16;
  const uint32_t e = (h16 >> 10) & 0x1fu;
  const uint32_t m = h16 & 0x3ffu;
  if (e == 0) {
    const float v = __fmul_rn((float)m, 0x1p-24f);  // subnormal: m * 2^-24, exact
    return __uint_as_float(__float_as_uint(v) | sign);
  }
  if (e == 31) return __uint_as_float(sign | 0x7f800000u | (m << 13));
  return __uint_as_float(sign | ((e + 112u) << 23) | (m << 13));
}

// fp32 -> binary16, round to nearest, ties to even, on the bit fields
// (subnormal halves included, whatever the hardware denormal mode).
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  const uint32_t x = __float_as_uint(f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax > 0x7f800000u) return sign | 0x7e00u | ((ax >> 13) & 0x3ffu);  // NaN stays NaN
  if (ax >= 0x477ff000u) return sign | 0x7c00u;                        // >= 65520 -> inf
  if (ax >= 0x38800000u) {                                             // normal half
    uint32_t m = ax - 0x38000000u;                                     // rebias 127 -> 15
    m += 0xfffu + ((m >> 13) & 1u);
    return sign | (m >> 13);
  }
  if (ax <= 0x33000000u) return sign;                                  // <= 2^-25 -> 0
  const uint32_t e = ax >> 23;                                         // 102..112
  const uint32_t mant = (ax & 0x7fffffu) | 0x800000u;
  const uint32_t sh = 126u - e;                                        // 14..24
  uint32_t q = mant >> sh;
  const uint32_t rem = mant & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1u);
  if (rem > half || (rem == half && (q & 1u))) ++q;                    // may carry into 2^-14
  return sign | q;
}

template <int DT>
struct Stor;
template <>
struct Stor<EMB_F32> {
  static constexpr int kBytes = 4;
};
template <>
struct Stor<EMB_BF16> {
  static constexpr int kBytes = 2;
};
template <>
struct Stor<EMB_F16> {
  static constexpr int kBytes = 2;
};

template <int DT>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
  if constexpr (DT == EMB_BF16) return bf16_to_f32(h);
  else return f16_to_f32(h);
}
template <int DT>
__device__ __forceinline__ uint32_t f32_to_half(float x) {
  if constexpr (DT == EMB_BF16) return f32_to_bf16_rne(x);
  else return f32_to_f16_rne(x);
}

// 16 bytes of storage -> 16/sizeof(S) floats.
template <int DT>
__device__ __forceinline__ void widen16(const u4 v, float* out) {
  if constexpr (DT == EMB_F32) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = half_to_f32<DT>(w[i] & 0xffffu);
      out[2 * i + 1] = half_to_f32<DT>(w[i] >> 16);
    }
  }
}

// Four consecutive elements of a row (16 bytes fp32 or 8 bytes 16-bit).
template <int DT>
__device__ __forceinline__ void load4(const void* p, float* out) {
  if constexpr (DT == EMB_F32) {
    const f4 v = *reinterpret_cast<const f4*>(p);
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  } else {
    const u2 v = *reinterpret_cast<const u2*>(p);
    out[0] = half_to_f32<DT>(v.x & 0xffffu);
    out[1] = half_to_f32<DT>(v.x >> 16);
    out[2] = half_to_f32<DT>(v.y & 0xffffu);
    out[3] = half_to_f32<DT>(v.y >> 16);
  }
}

template <int DT>
__device__ __forceinline__ void store4(void* p, const float* in) {
  if constexpr (DT == EMB_F32) {
    f4 v;
    v.x = in[0];
    v.y = in[1];
    v.z = in[2];
    v.w = in[3];
    *reinterpret_cast<f4*>(p) = v;
  } else {
    u2 v;
    v.x = f32_to_half<DT>(in[0]) | (f32_to_half<DT>(in[1]) << 16);
    v.y = f32_to_half<DT>(in[2]) | (f32_to_half<DT>(in[3]) << 16);
    *reinterpret_cast<u2*>(p) = v;
  }
}

// ---- index types ----------------------------------------------------------

template <typename IDX>
__device__ __forceinline__ long long ld_idx(const void* base, long long i) {
  return (long long)reinterpret_cast<const IDX*>(base)[i];
}

// ---- wave helpers -----------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << __lane_id()) - 1ull; }

// Blocks are handed to the 8 XCDs round-robin by block id; remap so that XCD
// x works on the contiguous range [x*n/8, (x+1)*n/8) of logical blocks and
// its private L2 sees one contiguous slice of the work. nblk_padded % 8 == 0.
__device__ __forceinline__ int xcd_remap(int bid, int nblk_padded) {
  const int per = nblk_padded >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Exclusive scan of one value per thread over a 256-thread block.
// `lds` needs 8 uint32 (4 waves). Returns the exclusive prefix; *total gets
// the block sum. Contains __syncthreads.
__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t v, uint32_t* lds, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  uint32_t wpre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t c = lds[w];
    if (w < wave) wpre += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return wpre + x - v;
}

// Table of a global key: the t with row_off[t] <= key < row_off[t+1], by
// binary search over the row offsets (staged in LDS by the caller).
__device__ __forceinline__ int table_of(const uint32_t* s_ro, int T, uint32_t key) {
  int lo = 0, hi = T;  // s_ro[lo] <= key < s_ro[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_ro[mid] <= key) lo = mid;
    else hi = mid;
  }
  return lo;
}

// ---- hash maps of the hash-keyed lookup (k_hash.hip, k_forward.hip) ----
constexpr long long kEmpty = (long long)0x8000000000000000ull;  // free slot; not a valid id

// SplitMix64's output mixer (Steele, Lea & Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Finds id in one table's map by linear probing from its mixed hash; with
// `insert`, claims the first free slot on the way with a 64-bit CAS (equal
// ids racing for one slot all end up on it). Returns the slot index, or -1
// (absent without insert; no free slot with it).
__device__ __forceinline__ long long find_slot(const HashMeta& m, unsigned long long* keys, long long id,
                                               bool insert) {
  uint32_t i = (uint32_t)mix64((uint64_t)id) & m.mask;
  for (uint32_t step = 0; step <= m.mask; ++step) {
    const long long slot = m.base + i;
    const long long k = (long long)__hip_atomic_load(keys + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k == id) return slot;
    if (k == kEmpty) {
      if (!insert) return -1;
      const unsigned long long old = atomicCAS(keys + slot, (unsigned long long)kEmpty, (unsigned long long)id);
      if ((long long)old == kEmpty || (long long)old == id) return slot;
    }
    i = (i + 1) & m.mask;
  }
  return -1;
}

}  // namespace emb
