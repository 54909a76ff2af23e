// route_kernels.h -- the router's small-T product and the per-token stable
// top-k as device functions (route.hip has the kernels, what they compute
// and where the pages say it).
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_r, a),
                                                 __builtin_bit_cast(bf16x8_r, b), c, 0, 0, 0);
}

constexpr int RS_WAVES = 8, RS_EXPERTS = 16;

// Logits of experts [e0, e0 + 16) for tokens [t0, min(T, t0 + 16 * MF)), by
// the 8 waves `wave` = 0..7 of a group (their partial tiles meet in `part`;
// the caller synchronizes the group between the two phases: sync()).  Each
// wave sums one eighth of K as an MFMA chain from zero in ascending K; the
// eight slices are then added in slice order.  U: K steps whose loads a wave
// issues before their MFMAs (registers; the sums do not depend on it).
template <int MF, int U = 10, typename Sync>
__device__ __forceinline__ void router_small_block(int T, int d, int E, const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int e0, int t0,
                                                   int wave, f32x4_t (&part)[RS_WAVES][MF][64],
                                                   Sync sync) {
  const int lane = threadIdx.x & 63;
  const int kw = d / RS_WAVES;  // multiple of 32 (d % 256 == 0)
  const int kb = wave * kw + 8 * (lane >> 4);
  const int er = e0 + (lane & 15);
  const uint16_t* bp = er < E ? wr + (size_t)er * d + kb : nullptr;
  const uint16_t* ap[MF];
#pragma unroll
  for (int m = 0; m < MF; m++) {
    const int t = t0 + m * 16 + (lane & 15);
    ap[m] = t < T ? x + (size_t)t * d + kb : nullptr;
  }
  f32x4_t acc[MF];
#pragma unroll
  for (int m = 0; m < MF; m++) acc[m] = f32x4_t{0, 0, 0, 0};
  const u32x4_t zero = {0, 0, 0, 0};
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
  sync();
  if (wave < MF) {  // wave m finishes token fragment m
    f32x4_t s = part[0][wave][lane];
#pragma unroll
    for (int w = 1; w < RS_WAVES; w++) s += part[w][wave][lane];
    const int e = e0 + (lane & 15);
    if (e < E) {
      const float bv = bias ? bias[e] : 0.0f;
      const int tq = t0 + wave * 16 + 4 * (lane >> 4);  // this lane's 4 token rows
      auto put = [&](int r) { logits[(size_t)(tq + r) * E + e] = s[r] + bv; };
      // all four rows in range: four stores behind one branch (a branch per
      // store makes each wait for the previous store to complete)
      if (tq + 3 < T) {
#pragma unroll
        for (int r = 0; r < 4; r++) put(r);
      } else {
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (tq + r < T) put(r);
      }
    }
  }
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

// One wave per token; 4 tokens per 256-thread block.  Expert e lives in lane
// e % 64, slot e / 64 (coalesced loads); PL slots a lane (8 for E <= 512, 16
// for E <= 1024).  Candidates are ordered by (key descending, expert id
// ascending); within a lane a lower slot is a lower id.  Each lane keeps its
// best and second-best remaining candidates.  Each of the k rounds takes a
// wave max of the lanes' best keys and -- only when several lanes hold that
// key -- a wave min of their expert ids, so equal logits go to the lower id.
// The winning lane marks the slot taken and promotes its second-best; a lane
// that wins again before its next scan rescans its slots (past the taken
// ones).  Per round that is a wave max, a ballot and a few moves in one lane,
// instead of a scan of every slot of the winner.

// Token t's logits, PL a lane (expert j * 64 + lane in slot j).  The loads
// carry no condition (slots past E re-read the row's last logit), so they
// issue back to back under one wait; a per-slot guarded load would wait for
// each in turn.
template <int PL>
__device__ __forceinline__ void topk_load(int t, int E, const float* __restrict__ logits,
                                          float (&lv)[PL]) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int j = 0; j < PL; j++) lv[j] = row[min(j * 64 + lane, E - 1)];
}

// Top-k and softmax of token t from its loaded logits; writes ids / w (and,
// if ids_lds is given, the ids at ids_lds[lds_row * k + s] too).
template <int PL>
__device__ __forceinline__ void topk_select(int t, int E, int k, const float (&lv)[PL],
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int32_t* ids_lds = nullptr, int lds_row = 0) {
  static_assert(PL <= 32, "the taken-slot mask is one dword");
  const int lane = threadIdx.x & 63;
  uint32_t key[PL];
#pragma unroll
  for (int j = 0; j < PL; j++) key[j] = j * 64 + lane < E ? order_key(lv[j]) : 0u;
  auto umax = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  auto umin = [](uint32_t x, uint32_t y) { return x < y ? x : y; };
  // the lane's best (bk, bj) and second-best (nk, nj) untaken candidates; a
  // strict > over ascending slots keeps the lower slot first among equal keys
  // (selects, no branches: every lane runs the same instructions)
  uint32_t bk = 0, nk = 0, taken = 0;
  int bj = 0, nj = 0;
  auto lane_top2 = [&]() __attribute__((always_inline)) {
    uint32_t k1 = 0, k2 = 0;
    int j1 = 0, j2 = 0;
#pragma unroll
    for (int j = 0; j < PL; j++) {
      const uint32_t kj = (taken >> j) & 1u ? 0u : key[j];
      const bool gt1 = kj > k1, gt2 = kj > k2;
      k2 = gt1 ? k1 : gt2 ? kj : k2;
      j2 = gt1 ? j1 : gt2 ? j : j2;
      k1 = gt1 ? kj : k1;
      j1 = gt1 ? j : j1;
    }
    bk = k1; bj = j1; nk = k2; nj = j2;
  };
  lane_top2();
  bool have2 = true;  // (nk, nj) is the true second-best since the last scan
  int my_id = 0;
  float my_logit = 0.0f, top_logit = 0.0f;
  for (int s = 0; s < k; s++) {
    const uint32_t m = wave_reduce_u32(bk, umax);
    const uint64_t holders = __ballot(bk == m);
    const uint32_t my_e = (uint32_t)(bj * 64 + lane);
    uint32_t e;
    if (__popcll(holders) == 1)
      e = (uint32_t)__builtin_amdgcn_readlane((int)my_e, __ffsll((long long)holders) - 1);
    else
      e = wave_reduce_u32(bk == m ? my_e : 0xFFFFFFFFu, umin);
    if (my_e == e) {  // the winning lane
      taken |= 1u << bj;
      if (have2) {  // its second-best (0: none left) moves up
        bk = nk;
        bj = nj;
        have2 = false;
      } else {  // it won twice since its last scan: rescan past the taken slots
        lane_top2();
        have2 = true;
      }
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
    if (ids_lds) ids_lds[lds_row * k + lane] = my_id;
  }
}

template <int PL>
__device__ __forceinline__ void topk_wave(int t, int E, int k, const float* __restrict__ logits,
                                          int32_t* __restrict__ ids, float* __restrict__ w) {
  float lv[PL];
  topk_load<PL>(t, E, logits, lv);
  topk_select<PL>(t, E, k, lv, ids, w);
}

}  // namespace moe
