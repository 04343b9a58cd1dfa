// Measurement aid, not part of the method: the read ceilings the path's
// kernels are compared with, and the ceiling of the fused update's mix of
// random row reads and writes. Every subgroup of 32 lanes reads rows of 512
// bytes (16 bytes per lane, one coalesced access, as a 128-column fp32 row
// of the upstream gradient is read) at pseudo-random row indices. With
// xcd_local, block b only reads rows of its eighth of the buffer: blocks are
// dealt round robin to the 8 XCDs, so each XCD's L2 serves its own eighth.
// Depending on the rows' footprint the reads are then served by the L2, by
// the MALL, or by HBM.
#include "emb_device.h"

namespace emb {

namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

constexpr int kProbeBlocks = 2048;

// LPR lanes per row: 32 for 512-byte rows, 16 for 256-byte rows.
template <int LPR>
__global__ __launch_bounds__(256) void k_probe_reads(const char* __restrict__ buf, uint32_t nrows,
                                                     uint32_t stride, int local, int reads,
                                                     float* __restrict__ sink) {
  const int lane = threadIdx.x & (LPR - 1);
  const uint32_t sg = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  uint32_t lo = 0, span = nrows;
  if (local) {
    span = nrows / 8;
    lo = (blockIdx.x & 7) * span;
  }
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < reads; it += 4) {
    f4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t row = lo + mix32(sg * 0x9E3779B1u + (uint32_t)(it + k) * 0x85EBCA77u) % span;
      v[k] = *reinterpret_cast<const f4*>(buf + (size_t)row * stride + lane * 16);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += v[k];
  }
  const float s = acc.x + acc.y + acc.z + acc.w;
  if (threadIdx.x == 0) sink[blockIdx.x] = s;  // keeps the loads
}

// The fused Adagrad update's access mix on rows of 512 bytes: per item, 3 (or
// 2) random source rows summed into a gradient, then one random row of `a`
// (weights) and of `b` (state) read, stepped and written back. Items that
// draw the same row race; the values written mean nothing.
__global__ __launch_bounds__(256) void k_probe_update(const float* __restrict__ src, uint32_t nsrc,
                                                      float* __restrict__ wa, float* __restrict__ wb,
                                                      uint32_t nrows, int items) {
  const int lane = threadIdx.x & 31;
  const int nsg = gridDim.x * 8;
  for (int i = blockIdx.x * 8 + (threadIdx.x >> 5); i < items; i += nsg) {
    const uint32_t row = mix32((uint32_t)i * 2654435761u + 17u) % nrows;
    const int nd = (i % 50) < 34 ? 3 : 2;
    float* pa = wa + (size_t)row * 128 + lane * 4;
    float* pb = wb + (size_t)row * 128 + lane * 4;
    const f4 w = *reinterpret_cast<const f4*>(pa);
    f4 s2 = *reinterpret_cast<const f4*>(pb);
    f4 v[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint32_t r = mix32((uint32_t)i * 0x9E3779B1u + (uint32_t)k * 0x85EBCA77u + 5u) % nsrc;
      v[k] = k < nd ? *reinterpret_cast<const f4*>(src + (size_t)r * 128 + lane * 4) : f4{0.f, 0.f, 0.f, 0.f};
    }
    const f4 g = v[0] + v[1] + v[2];
    s2 += g * g;
    f4 o;
    o.x = w.x - 0.01f * g.x / (sqrtf(s2.x) + 1e-8f);
    o.y = w.y - 0.01f * g.y / (sqrtf(s2.y) + 1e-8f);
    o.z = w.z - 0.01f * g.z / (sqrtf(s2.z) + 1e-8f);
    o.w = w.w - 0.01f * g.w / (sqrtf(s2.w) + 1e-8f);
    *reinterpret_cast<f4*>(pa) = o;
    *reinterpret_cast<f4*>(pb) = s2;
  }
}

}  // namespace

int probe_blocks() { return kProbeBlocks; }

hipError_t launch_probe_update(const float* src, uint32_t nsrc, float* a, float* b, uint32_t nrows, int items,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_probe_update, dim3(kProbeBlocks), dim3(256), 0, st, src, nsrc, a, b, nrows, items);
  return hipGetLastError();
}

hipError_t launch_probe_reads(const void* buf, uint32_t nrows, uint32_t stride, int local, int reads,
                              int row_bytes, float* sink, hipStream_t st) {
  if (row_bytes == 256)
    hipLaunchKernelGGL(k_probe_reads<16>, dim3(kProbeBlocks), dim3(256), 0, st, static_cast<const char*>(buf),
                       nrows, stride, local, reads, sink);
  else
    hipLaunchKernelGGL(k_probe_reads<32>, dim3(kProbeBlocks), dim3(256), 0, st, static_cast<const char*>(buf),
                       nrows, stride, local, reads, sink);
  return hipGetLastError();
}

}  // namespace emb
