// combine.hip -- fixed-order reduction of each token's routes, no atomics
// ("Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated prefill lane",
// step 5).  y[t] = ((o[inv[t*k]] + o[inv[t*k+1]]) + ... + o[inv[t*k+k-1]])
// + shared_out[t], summed in fp32 in exactly that order, then rounded to the
// output type.  One block per token; each thread owns 4 consecutive columns,
// so every load is a 16-byte fp32 vector and the sum order never depends on
// the launch shape.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

template <int ACT>
__global__ __launch_bounds__(128) void combine_kernel(int k, int d,
                                                      const float* __restrict__ out_assign,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ shared_out,
                                                      void* __restrict__ y) {
  __shared__ int rows[MAX_TOPK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) rows[threadIdx.x] = inv_perm[(size_t)t * k + threadIdx.x];
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += 128 * 4) {
    f32x4_t acc = *(const f32x4_t*)(out_assign + (size_t)rows[0] * d + c);
    for (int s = 1; s < k; s++) acc += *(const f32x4_t*)(out_assign + (size_t)rows[s] * d + c);
    if (shared_out) acc += *(const f32x4_t*)(shared_out + (size_t)t * d + c);
    if (ACT == MOE_F32) {
      *(f32x4_t*)((float*)y + (size_t)t * d + c) = acc;
    } else {
      uint2 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      *(uint2*)((uint16_t*)y + (size_t)t * d + c) = o;
    }
  }
}

hipError_t launch_combine(int T, int k, int d, int act, const float* out_assign,
                          const int32_t* inv_perm, const float* shared_out, void* y,
                          hipStream_t s) {
  if (act == MOE_F32)
    combine_kernel<MOE_F32><<<T, 128, 0, s>>>(k, d, out_assign, inv_perm, shared_out, y);
  else
    combine_kernel<MOE_BF16><<<T, 128, 0, s>>>(k, d, out_assign, inv_perm, shared_out, y);
  return hipGetLastError();
}

}  // namespace moe
