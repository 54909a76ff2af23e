// route.hip -- router logits and the deterministic stable top-k.
//
// Router: logits[t][e] = sum_i x[t][i] * Wr[e][i] (+ bias[e]), fp32 accumulate,
// the router weights kept unquantized ("Qwen3.8-Flash-Next-Dual-GPU" README,
// "Model artifact and memory placement": router preserved in BF16/F32).
// Top-k: one wave64 per token; k rounds of a wave-wide arg-max over 64-bit keys
// (order-preserving logit bits, then the complement of the expert id), so the
// larger logit wins and, among equal logits, the lower expert id -- the
// deterministic stable top-k of the README's "Independent decode lane".
// Routing weights: softmax over the k chosen logits.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- router GEMM
// Block tile 64 tokens x 64 experts, 4 waves in a 2x2 grid, each one 32x32
// MFMA tile; K streamed through LDS in chunks of 64.
constexpr int RT_M = 64, RT_N = 64;

__global__ __launch_bounds__(256) void router_bf16_kernel(int T, int d, int E,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[RT_M * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[RT_N * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * RT_M, n0 = blockIdx.x * RT_N;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc = {};
  // each thread stages two 16-byte pieces of A and two of B per chunk
  for (int kc = 0; kc < d; kc += 64) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      int piece = tid + j * 256;          // 0..511
      int r = piece >> 3, c = piece & 7;  // row 0..63, chunk 0..7
      u32x4_t va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
      if (m0 + r < T) va = *(const u32x4_t*)(x + (size_t)(m0 + r) * d + kc + c * 8);
      if (n0 + r < E) vb = *(const u32x4_t*)(wr + (size_t)(n0 + r) * d + kc + c * 8);
      *(u32x4_t*)(As + lds_a_index(r, c)) = va;
      *(u32x4_t*)(Bs + lds_a_index(r, c)) = vb;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; s++) {
      int c = 2 * s + (lane >> 5);
      u32x4_t a = *(const u32x4_t*)(As + lds_a_index(wm * 32 + (lane & 31), c));
      u32x4_t b = *(const u32x4_t*)(Bs + lds_a_index(wn * 32 + (lane & 31), c));
      acc = mfma32(a, b, acc);
    }
    __syncthreads();
  }
  const int col = n0 + wn * 32 + (lane & 31);
  if (col >= E) return;
  const float bv = bias ? bias[col] : 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row < T) logits[(size_t)row * E + col] = acc[r] + bv;
  }
}

// fp32 router: one thread per (token, expert), sequential fp32 dot product.
__global__ __launch_bounds__(64) void router_f32_kernel(int T, int d, int E,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ wr,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits) {
  int e = blockIdx.x * 64 + threadIdx.x, t = blockIdx.y;
  if (e >= E) return;
  const float* xr = x + (size_t)t * d;
  const float* wrow = wr + (size_t)e * d;
  float acc = 0.0f;
  for (int i = 0; i < d; i++) acc = fmaf(xr[i], wrow[i], acc);
  logits[(size_t)t * E + e] = acc + (bias ? bias[e] : 0.0f);
}

hipError_t launch_router_bf16(int T, int d, int E, const void* x, const void* wr, const float* bias,
                              float* logits, hipStream_t s) {
  dim3 grid((E + RT_N - 1) / RT_N, (T + RT_M - 1) / RT_M);
  router_bf16_kernel<<<grid, 256, 0, s>>>(T, d, E, (const uint16_t*)x, (const uint16_t*)wr, bias,
                                          logits);
  return hipGetLastError();
}

hipError_t launch_router_f32(int T, int d, int E, const float* x, const float* wr,
                             const float* bias, float* logits, hipStream_t s) {
  dim3 grid((E + 63) / 64, T);
  router_f32_kernel<<<grid, 64, 0, s>>>(T, d, E, x, wr, bias, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k
// Order-preserving map of a finite float to uint32 (larger float -> larger
// key); -0.0 is first made +0.0 so the two tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

constexpr int TOPK_PER_LANE = MAX_EXPERTS / 64;  // 16

// One wave per token; 4 tokens per 256-thread block.  Expert e lives in lane
// e % 64, slot e / 64 (coalesced loads).  A removed candidate has key 0, which
// no finite logit can produce (its low word is 0xFFFFFFFF - e > 0).
__global__ __launch_bounds__(256) void topk_kernel(int T, int E, int k,
                                                   const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nslot = (E + 63) >> 6;
  uint64_t key[TOPK_PER_LANE];
#pragma unroll
  for (int j = 0; j < TOPK_PER_LANE; j++) {
    int e = j * 64 + lane;
    key[j] = 0;
    if (j < nslot && e < E)
      key[j] = ((uint64_t)order_key(logits[(size_t)t * E + e]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
  }
  int my_id = 0;
  float my_logit = 0.0f, top_logit = 0.0f;
  for (int s = 0; s < k; s++) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < TOPK_PER_LANE; j++) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float lg = key_to_float((uint32_t)(best >> 32));
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < TOPK_PER_LANE; j++)
        if (j == (e >> 6)) key[j] = 0;
    }
    if (s == 0) top_logit = lg;
    if (s == lane) { my_id = e; my_logit = lg; }
  }
  const float ex = lane < k ? expf(my_logit - top_logit) : 0.0f;
  const float sum = wave_sum_f32(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_topk(int T, int E, int k, const float* logits, int32_t* ids, float* w,
                       hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(T, E, k, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
