// route.hip -- router logits and the deterministic stable top-k.
//
// Router: logits[t][e] = sum_i x[t][i] * Wr[e][i] (+ bias[e]), fp32 accumulate,
// the router weights kept unquantized ("Qwen3.8-Flash-Next-Dual-GPU" README,
// "Model artifact and memory placement": router preserved in BF16/F32).
// Top-k: one wave64 per token; k rounds of a wave-wide arg-max over
// order-preserving logit keys, equal keys resolved to the lower expert id --
// the deterministic stable top-k of the README's "Independent decode lane".
// Routing weights: softmax over the k chosen logits.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- router GEMM
// Two shapes, both bf16 MFMA with fp32 accumulation:
//  * small T (<= 64 tokens): one block per 16 experts, its 8 waves split K;
//    operands are read straight from global memory in MFMA fragment order
//    (16x16x32: lane l holds row l%16, K elements 8*(l/16)..+7), and the 8
//    partial 16x16 tiles are summed through LDS in a fixed wave order.
//  * large T: a block owns 64 tokens x 256 experts; the token rows are staged
//    through LDS (double-buffered, next chunk prefetched into registers) and
//    each wave streams its 64 router rows straight into MFMA registers.

typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_r, a),
                                                 __builtin_bit_cast(bf16x8_r, b), c, 0, 0, 0);
}

constexpr int RS_WAVES = 8, RS_EXPERTS = 16;

template <int MF>
__global__ __launch_bounds__(RS_WAVES * 64) void router_small_kernel(
    int T, int d, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits) {
  __shared__ f32x4_t part[RS_WAVES][MF][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * RS_EXPERTS;
  const int kw = d / RS_WAVES;  // multiple of 32 (d % 256 == 0)
  const int kb = wave * kw + 8 * (lane >> 4);
  const int er = e0 + (lane & 15);
  const uint16_t* bp = er < E ? wr + (size_t)er * d + kb : nullptr;
  const uint16_t* ap[MF];
#pragma unroll
  for (int m = 0; m < MF; m++) {
    const int t = m * 16 + (lane & 15);
    ap[m] = t < T ? x + (size_t)t * d + kb : nullptr;
  }
  f32x4_t acc[MF];
#pragma unroll
  for (int m = 0; m < MF; m++) acc[m] = f32x4_t{0, 0, 0, 0};
  const u32x4_t zero = {0, 0, 0, 0};
  constexpr int U = 10;  // K steps whose loads are all issued before their MFMAs
  for (int k0 = 0; k0 < kw; k0 += 32 * U) {
    u32x4_t bv[U], av[U][MF];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int k = k0 + 32 * u;
      const bool in = k < kw;
      bv[u] = (in && bp) ? *(const u32x4_t*)(bp + k) : zero;
#pragma unroll
      for (int m = 0; m < MF; m++) av[u][m] = (in && ap[m]) ? *(const u32x4_t*)(ap[m] + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int m = 0; m < MF; m++) acc[m] = mfma16(av[u][m], bv[u], acc[m]);
  }
#pragma unroll
  for (int m = 0; m < MF; m++) part[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave < MF) {  // wave m finishes token fragment m
    f32x4_t s = part[0][wave][lane];
#pragma unroll
    for (int w = 1; w < RS_WAVES; w++) s += part[w][wave][lane];
    const int e = e0 + (lane & 15);
    if (e < E) {
      const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = wave * 16 + 4 * (lane >> 4) + r;
        if (t < T) logits[(size_t)t * E + e] = s[r] + bv;
      }
    }
  }
}

constexpr int RL_M = 64, RL_N = 256;

__global__ __launch_bounds__(256, 2) void router_large_kernel(int T, int d, int E,
                                                              const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wr,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][RL_M * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * RL_M, n0 = blockIdx.x * RL_N + wave * 64;
  // A staging: 64 rows x 8 chunks of 16 B = 512 pieces, 2 per thread
  const int c8 = tid & 7;
  const uint16_t* arow[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int r = (tid >> 3) + 32 * j;
    arow[j] = m0 + r < T ? x + (size_t)(m0 + r) * d + c8 * 8 : nullptr;
  }
  // B: wave's 64 experts = 2 fragments of 32; lane l holds expert row l%32
  const uint16_t* brow[2];
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int e = n0 + f * 32 + (lane & 31);
    brow[f] = e < E ? wr + (size_t)e * d + 8 * (lane >> 5) : nullptr;
  }
  const u32x4_t zero = {0, 0, 0, 0};
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++) acc[i][0] = acc[i][1] = f32x16_t{};
  u32x4_t areg[2], b[2][4], bn[2][4];
  auto load_a = [&](int kc) {
#pragma unroll
    for (int j = 0; j < 2; j++) areg[j] = arow[j] ? *(const u32x4_t*)(arow[j] + kc) : zero;
  };
  auto store_a = [&](uint16_t* dst) {
#pragma unroll
    for (int j = 0; j < 2; j++) *(u32x4_t*)(dst + lds_a_index((tid >> 3) + 32 * j, c8)) = areg[j];
  };
  auto load_b = [&](int kc, u32x4_t (&dst)[2][4]) {
#pragma unroll
    for (int f = 0; f < 2; f++)
#pragma unroll
      for (int s = 0; s < 4; s++) dst[f][s] = brow[f] ? *(const u32x4_t*)(brow[f] + kc + s * 16) : zero;
  };
  auto compute = [&](const uint16_t* as, const u32x4_t (&bb)[2][4]) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const u32x4_t av = *(const u32x4_t*)(as + lds_a_index(i * 32 + (lane & 31), 2 * s + (lane >> 5)));
        acc[i][0] = mfma32(av, bb[0][s], acc[i][0]);
        acc[i][1] = mfma32(av, bb[1][s], acc[i][1]);
      }
    }
  };
  const int nk = d / 64;  // even (d % 256 == 0)
  load_a(0);
  load_b(0, b);
  store_a(As[0]);
  __syncthreads();
  for (int kc = 0; kc < nk; kc += 2) {
    load_a((kc + 1) * 64);
    load_b((kc + 1) * 64, bn);
    compute(As[0], b);
    store_a(As[1]);
    __syncthreads();
    if (kc + 2 < nk) {
      load_a((kc + 2) * 64);
      load_b((kc + 2) * 64, b);
    }
    compute(As[1], bn);
    if (kc + 2 < nk) store_a(As[0]);
    __syncthreads();
  }
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int e = n0 + f * 32 + (lane & 31);
    if (e >= E) continue;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int t = m0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) logits[(size_t)t * E + e] = acc[i][f][r] + bv;
      }
    }
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
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)wr;
  const int nb = (E + RS_EXPERTS - 1) / RS_EXPERTS;
  const int th = RS_WAVES * 64;
  if (T <= 16)
    router_small_kernel<1><<<nb, th, 0, s>>>(T, d, E, xp, wp, bias, logits);
  else if (T <= 32)
    router_small_kernel<2><<<nb, th, 0, s>>>(T, d, E, xp, wp, bias, logits);
  else if (T <= 64)
    router_small_kernel<4><<<nb, th, 0, s>>>(T, d, E, xp, wp, bias, logits);
  else
    router_large_kernel<<<dim3((E + RL_N - 1) / RL_N, (T + RL_M - 1) / RL_M), 256, 0, s>>>(
        T, d, E, xp, wp, bias, logits);
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
// key); -0.0 is first made +0.0 so the two tie.  No finite float maps to 0,
// which marks an absent or already chosen candidate.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Cross-lane steps inside a 16-lane row (DPP), then the four row results
// combined through scalar reads: every lane gets the same answer, and the
// combining order is fixed.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t a = __builtin_amdgcn_readlane((int)v, 0), b = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = __builtin_amdgcn_readlane((int)v, 32), d = __builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto add = [](uint32_t x, uint32_t y) { return __float_as_uint(__uint_as_float(x) + __uint_as_float(y)); };
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), add));
}

constexpr int TOPK_PER_LANE = MAX_EXPERTS / 64;  // 16

// One wave per token; 4 tokens per 256-thread block.  Expert e lives in lane
// e % 64, slot e / 64 (coalesced loads).  Each of the k rounds takes every
// lane's best remaining candidate (its lowest slot among equal keys), a wave
// max of those keys, and -- only when several lanes hold that key -- a wave
// min of their expert ids, so equal logits go to the lower id.
__global__ __launch_bounds__(256) void topk_kernel(int T, int E, int k,
                                                   const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint32_t key[TOPK_PER_LANE];
#pragma unroll
  for (int j = 0; j < TOPK_PER_LANE; j++) {
    const int e = j * 64 + lane;
    key[j] = e < E ? order_key(logits[(size_t)t * E + e]) : 0u;
  }
  auto umax = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  auto umin = [](uint32_t x, uint32_t y) { return x < y ? x : y; };
  int my_id = 0;
  float my_logit = 0.0f, top_logit = 0.0f;
  for (int s = 0; s < k; s++) {
    uint32_t bk = 0;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < TOPK_PER_LANE; j++)
      if (key[j] > bk) { bk = key[j]; bj = j; }
    const uint32_t m = wave_reduce_u32(bk, umax);
    const uint64_t holders = __ballot(bk == m);
    const uint32_t my_e = (uint32_t)(bj * 64 + lane);
    uint32_t e;
    if (__popcll(holders) == 1)
      e = (uint32_t)__builtin_amdgcn_readlane((int)my_e, __ffsll((long long)holders) - 1);
    else
      e = wave_reduce_u32(bk == m ? my_e : 0xFFFFFFFFu, umin);
    if (my_e == e) {
#pragma unroll
      for (int j = 0; j < TOPK_PER_LANE; j++)
        if (j == bj) key[j] = 0u;
    }
    const float lg = key_to_float(m);
    if (s == 0) top_logit = lg;
    if (s == lane) { my_id = (int)e; my_logit = lg; }
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
