// Host-only stand-ins for the kernel launchers of libkvattn, for the
// sanitizer build of the C ABI's host code (csrc/api.hip): every launcher
// reports that no device is present. Without a GPU no entry point reaches a
// launch (the device check comes first), so these only satisfy the linker.
#include <hip/hip_runtime.h>

#include "../../long_context_attention_paged_amd/csrc/launch.hpp"

namespace kvattn {

hipError_t launch_quantize(const float*, const float*, int64_t, int32_t, int32_t, const int32_t*,
                           int32_t, uint8_t*, uint8_t*, bool, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_summarize(const uint8_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                            int32_t, float*, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_score(const float*, const float*, int32_t, int32_t, int32_t, int32_t, double*,
                        hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_topk(const double*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t*,
                       hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode(const DecodeParams&, hipStream_t) { return hipErrorNoDevice; }
// the prefill kernel's rows per workgroup (8 waves x two 16-row tiles)
int32_t prefill_rows_per_tile() { return 256; }
hipError_t launch_prefill(const PrefillParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gather(const uint8_t*, const uint8_t*, const int32_t*, int32_t, int32_t,
                         const int32_t*, int32_t, int32_t, int32_t, uint8_t*, uint8_t*, int32_t*,
                         bool, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_rotate(float*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_merge(int32_t, int64_t, int32_t, const float*, const float*, float*, float*,
                        hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace kvattn
