// combine.hip -- fixed-order reduction of each token's routes, no atomics
// ("Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated prefill lane",
// step 5).  y[t] = ((o[inv[t*k]] + o[inv[t*k+1]]) + ... + o[inv[t*k+k-1]])
// + shared_out[t], summed in fp32 in exactly that order, then rounded to the
// output type.  Each thread owns 4 consecutive columns of one token, so every
// load is a 16-byte fp32 vector and the sum order never depends on the launch
// shape.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int COMBINE_COLS = 512;  // columns per block: 128 threads x 4

// Block (t, c): token t, columns [c*512, c*512 + 512).  A thread's k slot
// loads are issued eight at a time, then added in slot order.  Every partial
// is read exactly once: the loads are non-temporal.
template <int ACT>
__global__ __launch_bounds__(128) void combine_kernel(int k, int d,
                                                      const float* __restrict__ out_assign,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ shared_out,
                                                      void* __restrict__ y) {
  __shared__ int rows[MAX_TOPK];
  const int t = blockIdx.x;
  const int c = blockIdx.y * COMBINE_COLS + threadIdx.x * 4;
  if (threadIdx.x < k) rows[threadIdx.x] = inv_perm[(size_t)t * k + threadIdx.x];
  __syncthreads();
  if (c >= d) return;
  f32x4_t acc = __builtin_nontemporal_load((const f32x4_t*)(out_assign + (size_t)rows[0] * d + c));
  int s = 1;
  for (; s + 8 <= k; s += 8) {
    f32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = __builtin_nontemporal_load((const f32x4_t*)(out_assign + (size_t)rows[s + j] * d + c));
#pragma unroll
    for (int j = 0; j < 8; j++) acc += v[j];
  }
  for (; s < k; s++) acc += __builtin_nontemporal_load((const f32x4_t*)(out_assign + (size_t)rows[s] * d + c));
  if (shared_out) acc += __builtin_nontemporal_load((const f32x4_t*)(shared_out + (size_t)t * d + c));
  if (ACT == MOE_F32) {
    *(f32x4_t*)((float*)y + (size_t)t * d + c) = acc;
  } else {
    uint2 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    *(uint2*)((uint16_t*)y + (size_t)t * d + c) = o;
  }
}

hipError_t launch_combine(int T, int k, int d, int act, const float* out_assign,
                          const int32_t* inv_perm, const float* shared_out, void* y,
                          hipStream_t s) {
  const dim3 grid(T, (d + COMBINE_COLS - 1) / COMBINE_COLS);
  if (act == MOE_F32)
    combine_kernel<MOE_F32><<<grid, 128, 0, s>>>(k, d, out_assign, inv_perm, shared_out, y);
  else
    combine_kernel<MOE_BF16><<<grid, 128, 0, s>>>(k, d, out_assign, inv_perm, shared_out, y);
  return hipGetLastError();
}

}  // namespace moe
