// Stand-ins for everything the C-ABI host layer calls on the device side, so
// that emb_api.cpp can be built with the host sanitizers and driven without a
// GPU or a HIP runtime. The validation cases must never reach any of them:
// each one prints its name and aborts, which fails the harness.
#include <cstdio>
#include <cstdlib>

#include "emb_internal.h"

#define EMB_STUB_ABORT(name)                                                   \
  do {                                                                         \
    std::fprintf(stderr, "device-side call reached during validation: %s\n", name); \
    std::abort();                                                              \
  } while (0)

extern "C" {
hipError_t hipGetDevice(int*) { EMB_STUB_ABORT("hipGetDevice"); }
hipError_t hipMalloc(void**, size_t) { EMB_STUB_ABORT("hipMalloc"); }
hipError_t hipFree(void*) { EMB_STUB_ABORT("hipFree"); }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { EMB_STUB_ABORT("hipMemcpy"); }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  EMB_STUB_ABORT("hipMemcpyAsync");
}
hipError_t hipDeviceSynchronize(void) { EMB_STUB_ABORT("hipDeviceSynchronize"); }
hipError_t hipStreamSynchronize(hipStream_t) { EMB_STUB_ABORT("hipStreamSynchronize"); }
hipError_t hipEventCreate(hipEvent_t*) { EMB_STUB_ABORT("hipEventCreate"); }
hipError_t hipEventDestroy(hipEvent_t) { EMB_STUB_ABORT("hipEventDestroy"); }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { EMB_STUB_ABORT("hipEventRecord"); }
hipError_t hipEventSynchronize(hipEvent_t) { EMB_STUB_ABORT("hipEventSynchronize"); }
hipError_t hipEventElapsedTime(float*, hipEvent_t, hipEvent_t) { EMB_STUB_ABORT("hipEventElapsedTime"); }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace emb {
hipError_t launch_init_slice(const Geom&, const DevCtx&, int, int, int64_t, void*, float*, float*, uint64_t,
                             hipStream_t) {
  EMB_STUB_ABORT("launch_init_slice");
}
hipError_t launch_forward(const Geom&, const DevCtx&, const void*, const void*, int, long long, int, int, float*, int,
                          hipStream_t, const void*, long long, const HashView*) {
  EMB_STUB_ABORT("launch_forward");
}
hipError_t launch_gather_unique(const Geom&, const DevCtx&, const uint32_t*, const int32_t*, int, void*, hipStream_t) {
  EMB_STUB_ABORT("launch_gather_unique");
}
hipError_t launch_keys(const Geom&, const DevCtx&, const void*, const void*, int, long long, int, int,
                       const WsLayout&, char*, hipStream_t) {
  EMB_STUB_ABORT("launch_keys");
}
hipError_t launch_sort_hist(const SortPlan&, const SortBufs&, const uint64_t*, int, int, hipStream_t) {
  EMB_STUB_ABORT("launch_sort_hist");
}
hipError_t launch_sort_scan(const SortPlan&, const SortBufs&, int, hipStream_t) { EMB_STUB_ABORT("launch_sort_scan"); }
hipError_t launch_sort_scatter(const SortPlan&, const SortBufs&, const uint64_t*, uint64_t*, int, int, hipStream_t) {
  EMB_STUB_ABORT("launch_sort_scatter");
}
hipError_t launch_rle(const Geom&, int, const uint64_t*, int, int, const WsLayout&, char*, const RleOut&,
                      hipStream_t) {
  EMB_STUB_ABORT("launch_rle");
}
hipError_t launch_set_empty(const WsLayout&, char*, int32_t*, hipStream_t) { EMB_STUB_ABORT("launch_set_empty"); }
int probe_blocks() { return 2048; }
hipError_t launch_probe_reads(const void*, uint32_t, uint32_t, int, int, int, float*, hipStream_t) {
  EMB_STUB_ABORT("launch_probe_reads");
}
hipError_t launch_probe_update(const float*, uint32_t, float*, float*, uint32_t, int, hipStream_t) {
  EMB_STUB_ABORT("launch_probe_update");
}
hipError_t launch_reduce(const Geom&, const DevCtx&, int, int, int, int, const float*, const WsLayout&, const char*,
                         const uint32_t*, const int32_t*, float*, float, float, hipStream_t, const int32_t*) {
  EMB_STUB_ABORT("launch_reduce");
}
hipError_t launch_combine(const Geom&, const DevCtx&, int, int, const WsLayout&, const char*, const uint32_t*, float*,
                          float, float, hipStream_t, const int32_t*) {
  EMB_STUB_ABORT("launch_combine");
}
hipError_t launch_hash_clear(const HashView&, int, hipStream_t) { EMB_STUB_ABORT("launch_hash_clear"); }
hipError_t launch_hash_translate(const HashView&, const DevCtx&, int, const long long*, const void*, int, int, int,
                                 bool, const HashScratch&, void*, hipStream_t) {
  EMB_STUB_ABORT("launch_hash_translate");
}
hipError_t hash_noalloc_scratch(int, void**) { EMB_STUB_ABORT("hash_noalloc_scratch"); }
hipError_t launch_pack_dest(const Geom&, const DevCtx&, const int2*, int, int, const uint32_t*, const int32_t*,
                            uint64_t*, hipStream_t) {
  EMB_STUB_ABORT("launch_pack_dest");
}
hipError_t launch_pack_place(const uint64_t*, const uint32_t*, const int32_t*, int, int, uint32_t*, int32_t*,
                             hipStream_t) {
  EMB_STUB_ABORT("launch_pack_place");
}
hipError_t launch_pack_offsets(const uint64_t*, int, int, int32_t*, hipStream_t) {
  EMB_STUB_ABORT("launch_pack_offsets");
}
hipError_t launch_atomic_reduce(const Geom&, const void*, int, long long, int, int, const float*, const int32_t*,
                                const int32_t*, float*, hipStream_t) {
  EMB_STUB_ABORT("launch_atomic_reduce");
}
hipError_t launch_apply(const Geom&, const DevCtx&, int, int, const uint32_t*, const int32_t*, const float*, float,
                        float, hipStream_t) {
  EMB_STUB_ABORT("launch_apply");
}
}  // namespace emb
