// Host-only build of the library for the sanitizers (AddressSanitizer and
// UndefinedBehaviorSanitizer, see build.build_host_sanitized): api.cpp,
// split_policy.cpp and prefix_tree.cpp compiled by the host compiler, with
// the kernel launchers and the few HIP runtime calls api.cpp makes replaced
// by the stubs below, which report that there is no device. Every host path
// -- argument validation, window_safe_match, workspace sizing, the prefix
// tree -- runs unchanged; a call that would launch a kernel returns
// HA_ERR_HIP. Never part of the GPU library.
#include <hip/hip_runtime.h>

#include "../../include/ha_probe.h"
#include "kernels.hpp"
#include "status.hpp"

namespace ha {

hipError_t launch_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_read(const AppendArgs&, void*, void*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_verify(const VerifyArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t decode_scratch(int, void**) { return hipErrorNoDevice; }

}  // namespace ha

extern "C" {

const char* hipGetErrorString(hipError_t) { return "no device (host-only sanitizer build)"; }

hipError_t hipGetDevice(int* device) {
  if (device) *device = -1;
  return hipErrorNoDevice;
}

hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
  if (device) *device = -1;
  return hipErrorNoDevice;
}

// The measurement probes are kernels only: no host path to exercise.
ha_status ha_probe_paged_read(const ha_shape*, const ha_kv_view*, const int32_t*, int32_t, uint32_t*, int32_t,
                              void*) {
  return ha::set_error(HA_ERR_HIP, "no device (host-only sanitizer build)");
}

ha_status ha_probe_mfma_bf16(int32_t, int32_t, float*, void*) {
  return ha::set_error(HA_ERR_HIP, "no device (host-only sanitizer build)");
}

ha_status ha_probe_coissue(int32_t, int32_t, int32_t, float*, void*) {
  return ha::set_error(HA_ERR_HIP, "no device (host-only sanitizer build)");
}

}  // extern "C"
