// noalloc.hip -- moe_grouped_ffn_noalloc: moe_grouped_ffn for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its scratch -- the row-tile plan,
// the intermediate h, the fp16 (or MXFP4) copy of the activations -- lives in
// one file-scope device array instead of a caller's workspace, laid out as
// moe_workspace_bytes lays out a workspace.  The row-tile plan is rebuilt from
// the caller's offsets, so no moe_permute workspace is needed either.
//
// Each GPU the library runs on holds its own copy of the array (8 MiB) until
// the process ends.  Every call on a GPU uses that GPU's copy: calls that
// overlap on one GPU (two streams, two threads) race on it and must be
// serialized by the caller.  Nothing in it has to start at zero -- every byte
// a call reads was written earlier in the same call.
#include <mutex>

#include "moe_internal.h"

namespace moe {
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(8) << 20;
}

static __device__ __align__(256) uint8_t scratch[moe::NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES];  // device address of `scratch` on each GPU

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current.  (Host code never uses the array's own
// name as an address: on the host it is only a stand-in for the symbol.)
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_grouped_ffn_noalloc(const moe_desc* desc, int32_t T, int32_t k,
                                              const void* hidden, const float* topk_w,
                                              const int32_t* offsets, const int32_t* perm,
                                              const void* routed_blob, const void* shared_blob,
                                              float* out_assign, float* shared_out,
                                              void* stream) {
  return moe::grouped_ffn_call(desc, T, k, hidden, topk_w, offsets, perm, routed_blob,
                               shared_blob, out_assign, shared_out, nullptr,
                               moe::NOALLOC_SCRATCH_BYTES, scratch_of_current_device, stream);
}
