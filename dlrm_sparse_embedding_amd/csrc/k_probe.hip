// Measurement aid, not part of the method: the read ceilings the path's
// kernels are compared with. Every subgroup of 32 lanes reads rows of 512
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

__global__ __launch_bounds__(256) void k_probe_reads(const char* __restrict__ buf, uint32_t nrows,
                                                     uint32_t stride, int local, int reads,
                                                     float* __restrict__ sink) {
  const int lane = threadIdx.x & 31;
  const uint32_t sg = blockIdx.x * 8 + (threadIdx.x >> 5);
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

}  // namespace

int probe_blocks() { return kProbeBlocks; }

hipError_t launch_probe_reads(const void* buf, uint32_t nrows, uint32_t stride, int local, int reads,
                              float* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_probe_reads, dim3(kProbeBlocks), dim3(256), 0, st, static_cast<const char*>(buf), nrows,
                     stride, local, reads, sink);
  return hipGetLastError();
}

}  // namespace emb
