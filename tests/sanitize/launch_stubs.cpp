// launch_stubs.cpp -- stand-ins for the kernel launches of the HIP library, so
// that its host side (abi.cpp: argument checks, blob packing and unpacking,
// workspace sizing) can be built by the host compiler alone, with address and
// undefined-behaviour sanitizers, and driven by the host tests.  No test that
// runs against this build reaches a launch; if one did, it gets an error back.
#include "../../expert_grouped_quantized_amd/csrc/moe_internal.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "no device in the host-only build"; }

namespace moe {
hipError_t launch_router_bf16(int, int, int, const void*, const void*, const float*, float*,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_router_f32(int, int, int, const float*, const float*, const float*, float*,
                             hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_topk(int, int, int, const float*, int32_t*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_plan(int, int, int, const int32_t*, int32_t*, int32_t*, int32_t*, void*,
                       const WsLayout&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_ffn_bf16(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_ffn_f32(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_ffn_lowbit(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_ffn_mx(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_x_to_f16(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_combine(int, int, int, int, const float*, const int32_t*, const float*, void*,
                          hipStream_t) {
  return hipErrorNoDevice;
}
}  // namespace moe
