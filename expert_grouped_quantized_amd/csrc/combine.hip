// combine.hip -- fixed-order reduction of each token's routes, no atomics
// ("Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated prefill lane",
// step 5).  y[t] = ((o[inv[t*k]] + o[inv[t*k+1]]) + ... + o[inv[t*k+k-1]])
// + shared_out[t], summed in fp32 in exactly that order (0 + o[...] first,
// which is exact), then rounded to the output type.  One block per token; each
// thread owns a run of consecutive columns, so the sum order never depends on
// the launch shape.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// act F32: fp32 partials, 4 columns per thread (16-byte loads).
// act BF16: bf16 partials, 8 columns per thread (16-byte loads), widened to
// fp32 before the sum.
template <int ACT>
__global__ __launch_bounds__(128) void combine_kernel(int k, int d, const void* __restrict__ out_assign,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const void* __restrict__ shared_out,
                                                      void* __restrict__ y) {
  __shared__ int rows[MAX_TOPK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) rows[threadIdx.x] = inv_perm[(size_t)t * k + threadIdx.x];
  __syncthreads();
  if (ACT == MOE_F32) {
    const float* oa = (const float*)out_assign;
    const float* so = (const float*)shared_out;
    for (int c = threadIdx.x * 4; c < d; c += 128 * 4) {
      f32x4_t acc = *(const f32x4_t*)(oa + (size_t)rows[0] * d + c);
      for (int s = 1; s < k; s++) acc += *(const f32x4_t*)(oa + (size_t)rows[s] * d + c);
      if (so) acc += *(const f32x4_t*)(so + (size_t)t * d + c);
      *(f32x4_t*)((float*)y + (size_t)t * d + c) = acc;
    }
  } else {
    const uint16_t* oa = (const uint16_t*)out_assign;
    const uint16_t* so = (const uint16_t*)shared_out;
    auto add8 = [](float (&acc)[8], const u32x4_t& v) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        acc[2 * j] += bf16_lo(v[j]);
        acc[2 * j + 1] += bf16_hi(v[j]);
      }
    };
    for (int c = threadIdx.x * 8; c < d; c += 128 * 8) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int s = 0; s < k; s++) add8(acc, *(const u32x4_t*)(oa + (size_t)rows[s] * d + c));
      if (so) add8(acc, *(const u32x4_t*)(so + (size_t)t * d + c));
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; j++) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
      *(u32x4_t*)((uint16_t*)y + (size_t)t * d + c) = o;
    }
  }
}

hipError_t launch_combine(int T, int k, int d, int act, const void* out_assign,
                          const int32_t* inv_perm, const void* shared_out, void* y,
                          hipStream_t s) {
  if (act == MOE_F32)
    combine_kernel<MOE_F32><<<T, 128, 0, s>>>(k, d, out_assign, inv_perm, shared_out, y);
  else
    combine_kernel<MOE_BF16><<<T, 128, 0, s>>>(k, d, out_assign, inv_perm, shared_out, y);
  return hipGetLastError();
}

}  // namespace moe
