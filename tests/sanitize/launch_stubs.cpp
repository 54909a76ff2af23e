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
hipError_t launch_plan(int, int, int, int, const int32_t*, int32_t*, int32_t*, int32_t*, void*,
                       const WsLayout&, int, const uint16_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_route_plan_small(int, int, int, int, const void*, const void*, const float*,
                                   float*, int32_t*, float*, int32_t*, int32_t*, int32_t*, int,
                                   void*, const WsLayout&, bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_ffn_bf16(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_ffn_f32(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_ffn_lowbit(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_ffn_mx(const FfnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_combine(int, int, int, int, const float*, const int32_t*, const float*, void*,
                          hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_tiles_from_offsets(int, int, int, const int32_t*, int4*, int, int,
                                     const uint16_t*, uint16_t*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
}  // namespace moe

// The no-allocation entry point of noalloc.hip (a device-side source): the
// same host checks, with a scratch lookup that reports no device.
static hipError_t no_scratch(void**) { return hipErrorNoDevice; }
extern "C" moe_status moe_grouped_ffn_noalloc(const moe_desc* desc, int32_t T, int32_t k,
                                              const void* hidden, const float* topk_w,
                                              const int32_t* offsets, const int32_t* perm,
                                              const void* routed_blob, const void* shared_blob,
                                              float* out_assign, float* shared_out,
                                              void* stream) {
  return moe::grouped_ffn_call(desc, T, k, hidden, topk_w, offsets, perm, routed_blob,
                               shared_blob, out_assign, shared_out, nullptr, size_t(8) << 20,
                               no_scratch, stream);
}
