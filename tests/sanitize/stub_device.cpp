// Host-only stand-ins for the device side of libds4q.so, so that the ABI's
// host code (abi.cpp) can be built and run on a machine without a GPU under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every kernel launcher
// records its call and returns success without touching the (fake) device
// pointers; the HIP runtime calls abi.cpp makes are no-ops on host memory.
// Test infrastructure only: never part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../bit_quantized_moe_q2_amd/csrc/launch.h"
#include "../../include/ds4q.h"

long g_launches = 0;

namespace ds4q {
#define STUB(...) { (void)sizeof(#__VA_ARGS__); ++g_launches; return hipSuccess; }
hipError_t launch_dequant(int, const void *, int64_t, int64_t, bool, void *, hipStream_t) STUB()
hipError_t launch_matvec(int, const void *, int64_t, int64_t, const float *, int, float *, hipStream_t) STUB()
hipError_t launch_topk(const float *, int, int, int, const float *, int, float, const RouteBufs &, hipStream_t) STUB()
hipError_t launch_group(int, int, int, int, bool, const RouteBufs &, hipStream_t) STUB()
hipError_t launch_decode_q2k_t1(const MoeDims &, const float *, const float *, bool, float, const RouteBufs &,
                                float *, float *, bool, int, const SteerArgs &, hipStream_t) STUB()
hipError_t launch_decode_q41_t1(const MoeDims &, const float *, const float *, bool, float, const RouteBufs &,
                                float *, float *, bool, int, const SteerArgs &, hipStream_t) STUB()
hipError_t launch_combine(const float *, const RouteBufs &, int, int, int, bool, float *, bool, const SteerArgs &,
                          hipStream_t) STUB()
hipError_t launch_combine(const uint16_t *, const RouteBufs &, int, int, int, bool, float *, bool,
                          const SteerArgs &, hipStream_t) STUB()
hipError_t launch_prep_f16(const void *, bool, bool, const float *, int64_t, int, int, const PrepF16 &, hipStream_t) STUB()
hipError_t launch_prefill_f16_gateup(const MoeDims &, const PrepF16 &, int, const RouteBufs &, int, uint16_t *,
                                     hipStream_t) STUB()
hipError_t launch_prefill_f16_down(const MoeDims &, const PrepF16 &, int, const RouteBufs &, int, uint16_t *,
                                   hipStream_t) STUB()
hipError_t launch_prep_d3(const float *, const float *, int64_t, int, int, const PrepD3 &, hipStream_t) STUB()
hipError_t launch_decode_grouped(const MoeDims &, const PrepD3 &, int, const RouteBufs &, int, float *, int,
                                 hipStream_t) STUB()
hipError_t launch_steer(const float *, float, const float *, int64_t, int, float *, bool, hipStream_t) STUB()
hipError_t launch_act_encode(const float *, int64_t, int, void *, hipStream_t) STUB()
hipError_t launch_act_decode(const void *, int64_t, int, float *, hipStream_t) STUB()
hipError_t launch_imatrix(const MoeDims &, const RouteBufs &, int, int, const ImatRows &, float *,
                          const ImatRows &, float *, float *, hipStream_t) STUB()
static unsigned char g_scratch[DS4Q_SCRATCH_BYTES];
hipError_t scratch_address(void **out) { *out = g_scratch; return hipSuccess; }

// the workspace layout of the prep rows (as in the library)
size_t prep_f16_bytes(int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return up((size_t)rows * K * 2) + up((size_t)rows * 4);
}
PrepF16 prep_f16_view(void *base, int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  uint8_t *b = static_cast<uint8_t *>(base);
  PrepF16 p;
  p.q = reinterpret_cast<uint16_t *>(b);
  p.sig = reinterpret_cast<float *>(b + up((size_t)rows * K * 2));
  return p;
}
size_t prep_d3_bytes(int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return up((size_t)rows * (K / 256) * 768) + up((size_t)rows * 4) + up((size_t)rows * (K / 32) * 4);
}
PrepD3 prep_d3_view(void *base, int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  PrepD3 p;
  p.q = static_cast<uint8_t *>(base);
  p.sig = reinterpret_cast<float *>(p.q + up((size_t)rows * (K / 256) * 768));
  p.xs = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(p.sig) + up((size_t)rows * 4));
  return p;
}
}  // namespace ds4q

// HIP runtime calls of abi.cpp on host memory.
struct StubEvent { int recorded; };
extern "C" {
hipError_t hipEventCreate(hipEvent_t *e) { *e = reinterpret_cast<hipEvent_t>(new StubEvent{0}); return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) { delete reinterpret_cast<StubEvent *>(e); return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) { reinterpret_cast<StubEvent *>(e)->recorded = 1; return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t e) { return reinterpret_cast<StubEvent *>(e)->recorded ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t a, hipEvent_t b) {
  *ms = 0.001f;
  return reinterpret_cast<StubEvent *>(a)->recorded && reinterpret_cast<StubEvent *>(b)->recorded ? hipSuccess : hipErrorInvalidValue;
}
// the copies of routing outputs move between host stand-ins of device buffers
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t) {
  memmove(dst, src, n);
  return hipSuccess;
}
}
