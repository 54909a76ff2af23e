// route.hip -- router logits and the deterministic stable top-k.
//
// Router: logits[t][e] = sum_i x[t][i] * Wr[e][i] (+ bias[e]), fp32 accumulate,
// the router weights kept unquantized ("Qwen3.8-Flash-Next-Dual-GPU" README,
// "Model artifact and memory placement": router preserved in BF16/F32).
// Top-k: one wave64 per token; k rounds of a wave-wide arg-max over
// order-preserving logit keys, equal keys resolved to the lower expert id --
// the deterministic stable top-k of the README's "Independent decode lane".
// Routing weights: softmax over the k chosen logits.
#include "route_kernels.h"

namespace moe {

// ---------------------------------------------------------------- router GEMM
// Two shapes, both bf16 MFMA with fp32 accumulation:
//  * small T (<= 64 tokens): one block per 16 experts, its 8 waves split K;
//    operands are read straight from global memory in MFMA fragment order
//    (16x16x32: lane l holds row l%16, K elements 8*(l/16)..+7), and the 8
//    partial 16x16 tiles are summed through LDS in a fixed wave order.
//  * large T: a block (8 waves) owns 64 tokens x 128 experts; token rows and
//    router rows are both staged through LDS with four chunks of loads in
//    flight.

template <int MF>
__global__ __launch_bounds__(RS_WAVES * 64) void router_small_kernel(
    int T, int d, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits) {
  __shared__ f32x4_t part[RS_WAVES][MF][64];
  router_small_block<MF>(T, d, E, x, wr, bias, logits, blockIdx.x * RS_EXPERTS, 0,
                         threadIdx.x >> 6, part, [] { __syncthreads(); });
}

constexpr int RL_M = 64, RL_N = 128, RL_LEAD = 4;

// Large T: a block owns 64 tokens x 128 experts; each of its 8 waves makes
// 32 tokens x 32 experts (two waves per SIMD: one wave's LDS reads and
// barrier waits overlap the other's MFMAs; measured 4 us faster at T=4096
// than 4 waves of 64 x 32).  A logit is summed exactly as the small-T kernel
// sums it -- K in eight equal slices, each an MFMA chain from zero in
// ascending K, the slices then added in slice order -- so a token's logits,
// and hence its routing, do not depend on how many tokens share the call.
// Token rows and router rows are both staged through LDS, 64 K at a time, in
// four slots: step c computes chunk c from slot c % 4 and stores chunk c + 2
// into slot (c + 2) % 4, with a barrier after every second step (-1.3 us at
// T=4096 against two slots and a barrier a step); every thread keeps RL_LEAD
// chunks of its staging loads in flight (issued in the order they are waited
// for, no load behind a condition).  Rows past T or E read row T-1 / E-1 and are
// never stored.  Grid: the expert blocks of one token block share an XCD
// (block b runs on XCD b % 8), so its L2 holds their common token rows.
__global__ __launch_bounds__(512, 1) void router_large_kernel(int T, int d, int E, int neb,
                                                              int ntb,
                                                              const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wr,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[4][RL_M * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[4][RL_N * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int th = wave & 1, eq = wave >> 1;  // token half, expert quarter
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  const int tb = (j / neb) * 8 + xcd, eb = j % neb;
  if (tb >= ntb) return;
  const int m0 = tb * RL_M, n0 = eb * RL_N;
  // staging pieces (16 B): A 64 rows x 8 = 512 -> 1 per thread, B 128 x 8 -> 2
  const int c8 = tid & 7, r0 = tid >> 3;  // r0 in 0..63
  const uint16_t* ap = x + (size_t)min(m0 + r0, T - 1) * d + c8 * 8;
  const uint16_t* bp[2];
#pragma unroll
  for (int q = 0; q < 2; q++) bp[q] = wr + (size_t)min(n0 + r0 + 64 * q, E - 1) * d + c8 * 8;
  u32x4_t ar[RL_LEAD], br[RL_LEAD][2];
  auto load = [&](int kc, u32x4_t& a, u32x4_t (&bb)[2]) {
    a = *(const u32x4_t*)(ap + kc * 64);
#pragma unroll
    for (int q = 0; q < 2; q++) bb[q] = *(const u32x4_t*)(bp[q] + kc * 64);
  };
  auto store = [&](int buf, const u32x4_t& a, const u32x4_t (&bb)[2]) {
    *(u32x4_t*)(As[buf] + lds_a_index(r0, c8)) = a;
#pragma unroll
    for (int q = 0; q < 2; q++) *(u32x4_t*)(Bs[buf] + lds_a_index(r0 + 64 * q, c8)) = bb[q];
  };
  f32x4_t acc[2][2], tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
    acc[i][0] = acc[i][1] = tot[i][0] = tot[i][1] = f32x4_t{0, 0, 0, 0};
  const int slice_steps = d / (32 * RS_WAVES);  // 32-K steps per K slice
  auto compute = [&](int buf, int kc) {
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int ch = 4 * s + (lane >> 4);
      u32x4_t bv[2];
#pragma unroll
      for (int f = 0; f < 2; f++)
        bv[f] = *(const u32x4_t*)(Bs[buf] + lds_a_index(eq * 32 + f * 16 + (lane & 15), ch));
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const u32x4_t av = *(const u32x4_t*)(As[buf] + lds_a_index(th * 32 + i * 16 + (lane & 15), ch));
        acc[i][0] = mfma16(av, bv[0], acc[i][0]);
        acc[i][1] = mfma16(av, bv[1], acc[i][1]);
      }
      const int step = 2 * kc + s + 1;
      if (step % slice_steps == 0) {
        const bool first = step == slice_steps;
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int f = 0; f < 2; f++) {
            tot[i][f] = first ? acc[i][f] : tot[i][f] + acc[i][f];
            acc[i][f] = f32x4_t{0, 0, 0, 0};
          }
      }
    }
  };
  const int nk = d / 64;
#pragma unroll
  for (int p = 0; p < RL_LEAD; p++) load(p, ar[p], br[p]);
  store(0, ar[0], br[0]);
  store(1, ar[1], br[1]);
  __syncthreads();
  for (int kc0 = 0; kc0 < nk - RL_LEAD; kc0 += RL_LEAD) {
#pragma unroll
    for (int p = 0; p < RL_LEAD; p++) {
      load(kc0 + p + RL_LEAD, ar[p], br[p]);
      compute(p, kc0 + p);
      store((p + 2) % 4, ar[(p + 2) % RL_LEAD], br[(p + 2) % RL_LEAD]);
      if (p & 1) __syncthreads();
    }
  }
#pragma unroll
  for (int p = 0; p < RL_LEAD; p++) {
    compute(p, nk - RL_LEAD + p);
    if (p < 2) store(p + 2, ar[p + 2], br[p + 2]);
    if (p == 1) __syncthreads();
  }
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int e = n0 + eq * 32 + f * 16 + (lane & 15);
    if (e >= E) continue;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = m0 + th * 32 + i * 16 + 4 * (lane >> 4) + r;
        if (t < T) logits[(size_t)t * E + e] = tot[i][f][r] + bv;
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
  else {
    const int neb = (E + RL_N - 1) / RL_N, ntb = (T + RL_M - 1) / RL_M;
    const int blocks = (ntb + 7) / 8 * 8 * neb;
    router_large_kernel<<<blocks, 512, 0, s>>>(T, d, E, neb, ntb, xp, wp, bias, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_f32(int T, int d, int E, const float* x, const float* wr,
                             const float* bias, float* logits, hipStream_t s) {
  dim3 grid((E + 63) / 64, T);
  router_f32_kernel<<<grid, 64, 0, s>>>(T, d, E, x, wr, bias, logits);
  return hipGetLastError();
}

// One wave per token, 4 tokens per 256-thread block (topk_wave).
template <int PL>
__global__ __launch_bounds__(256) void topk_kernel(int T, int E, int k,
                                                   const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave<PL>(t, E, k, logits, ids, w);
}

hipError_t launch_topk(int T, int E, int k, const float* logits, int32_t* ids, float* w,
                       hipStream_t s) {
  static_assert(MAX_EXPERTS <= 16 * 64, "top-k holds at most 16 candidates a lane");
  if (E <= 8 * 64)
    topk_kernel<8><<<(T + 3) / 4, 256, 0, s>>>(T, E, k, logits, ids, w);
  else
    topk_kernel<16><<<(T + 3) / 4, 256, 0, s>>>(T, E, k, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
