// Host-only stand-ins for the kernel launchers, linked with the C ABI's host
// code (wq_api.hip, wq_plan.cpp) into a sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer) that the CPU tests load in place of libwq.so.
// Every launcher counts the attempt and fails the way the real library does
// on a machine without a GPU (hipErrorNoDevice), so a call that passes the
// host checks reports WQ_EHIP; the counter shows whether a rejected call
// enqueued anything before it failed.
#include <hip/hip_runtime_api.h>

#include <atomic>

#include "wq_internal.hpp"

namespace {
std::atomic<long> g_launches{0};
hipError_t attempt() {
  g_launches.fetch_add(1);
  return hipErrorNoDevice;
}
}  // namespace

extern "C" long wq_hostcheck_launches(void) { return g_launches.load(); }

extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "no device (host check build)"; }

namespace wq {
hipError_t launch_linear(int, const LinearArgs&, const LinearPlan&, hipStream_t) { return attempt(); }
hipError_t launch_gemm_tiled(int, const LinearArgs&, const LinearPlan&, hipStream_t) { return attempt(); }
hipError_t launch_gemm_mid(int, const LinearArgs&, hipStream_t) { return attempt(); }
hipError_t launch_quantize(int, const uint16_t*, int64_t, int64_t, void*, void*, float*, hipStream_t) { return attempt(); }
hipError_t launch_read_stream(const void*, size_t, uint32_t*, hipStream_t) { return attempt(); }
hipError_t launch_pack(int, const uint8_t*, int64_t, int64_t, uint8_t*, hipStream_t) { return attempt(); }
hipError_t launch_dequantize(int, int, const void*, const void*, const float*, int64_t, int64_t, uint16_t*, hipStream_t) {
  return attempt();
}
hipError_t launch_repack(int, int64_t, int64_t, int, const void*, const void*, int, void*, void*, hipStream_t) {
  return attempt();
}
hipError_t launch_absmax(const uint16_t*, int64_t, float*, hipStream_t) { return attempt(); }
hipError_t launch_fp8_scale(const float*, float*, int64_t, hipStream_t) { return attempt(); }
hipError_t launch_quantize_act(const uint16_t*, int64_t, const float*, uint8_t*, hipStream_t) { return attempt(); }
hipError_t launch_static_mlp2(const Mlp2Args&, hipStream_t) { return attempt(); }
hipError_t launch_mx_quantize_act(const uint16_t*, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) { return attempt(); }
hipError_t launch_mx_linear(const LinearArgs&, hipStream_t) { return attempt(); }
hipError_t launch_f8_gemm_tiled(const LinearArgs&, hipStream_t) { return attempt(); }
hipError_t noalloc_scratch(void**) { return attempt(); }
}  // namespace wq
