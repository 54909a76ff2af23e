// ffn.hip -- expert-grouped SwiGLU GEMMs ("Qwen3.8-Flash-Next-Dual-GPU"
// README, section "Dedicated prefill lane", steps 2-4).
//
// Work unit: one row tile (up to BM = 128 consecutive rows of one expert's
// group in the route plan, or 128 tokens of the always-active shared expert)
// times one column block.  A block is 4 wave64s:
//   stage 1: h[p] = w_p * silu(Wg x_t) (.) (Wu x_t)   -> h (bf16), rows p
//            each wave owns 32 h columns: 32 gate rows and 32 up rows of W1
//   stage 2: out[p] = Wd h[p]                          -> fp32, one row per
//            assignment (out_assign) or per token (shared_out)
//            each wave owns 64 output columns
// Activations (x rows gathered through perm, or h rows) are staged through
// LDS, 64 K at a time, double-buffered, and read as MFMA A operands by all 4
// waves.  Weights stream straight from HBM into each wave's registers in the
// tile order moe_pack_experts wrote them (one contiguous run per wave), are
// dequantized in registers to bf16 (int4: code * fp16 group scale, rounded to
// nearest even; int8: the exact code, its row scale applied to the fp32
// accumulator), and feed bf16 MFMA 32x32x16 with fp32 accumulation.  A wave
// covers all rows of its tile, so each weight is read and dequantized once per
// row tile.  Row tiles with fewer than 128 rows skip their empty 32-row MFMA
// fragments.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// ---- weight registers of one wave tile (64 rows x 64 K) -------------------
template <int FMT>
struct WTile;

template <>
struct WTile<MOE_BF16> {
  u32x4_t v[8];  // [frag][step]
  __device__ __forceinline__ void load(const uint8_t* t, int lane) {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = ((const u32x4_t*)t)[j * 64 + lane];
  }
  __device__ __forceinline__ u32x4_t frag(int f, int s) const { return v[f * 4 + s]; }
};

template <>
struct WTile<MOE_I4_G32> {
  u32x4_t v[2];  // [frag], component = step; nibbles hold code + 8
  uint2 sc;      // fp16 scales: frag0 group0, frag0 group1, frag1 group0, frag1 group1
  __device__ __forceinline__ void load(const uint8_t* t, int lane) {
    v[0] = ((const u32x4_t*)t)[lane];
    v[1] = ((const u32x4_t*)t)[64 + lane];
    sc = ((const uint2*)(t + 2048))[lane & 31];
  }
  __device__ __forceinline__ u32x4_t frag(int f, int s) const {
    const uint32_t word = f ? (s < 2 ? sc.y & 0xffffu : sc.y >> 16) : (s < 2 ? sc.x & 0xffffu : sc.x >> 16);
    const float scale = f16_bits_to_f32((uint16_t)word);
    const float bias = -8.0f * scale;
    const uint32_t q = v[f][s];
    const uint32_t lo = q & 0x0f0f0f0fu, hi = (q >> 4) & 0x0f0f0f0fu;
    u32x4_t r;
    r[0] = pack_bf16x2(fmaf((float)(lo & 0xff), scale, bias), fmaf((float)(hi & 0xff), scale, bias));
    r[1] = pack_bf16x2(fmaf((float)((lo >> 8) & 0xff), scale, bias),
                       fmaf((float)((hi >> 8) & 0xff), scale, bias));
    r[2] = pack_bf16x2(fmaf((float)((lo >> 16) & 0xff), scale, bias),
                       fmaf((float)((hi >> 16) & 0xff), scale, bias));
    r[3] = pack_bf16x2(fmaf((float)(lo >> 24), scale, bias), fmaf((float)(hi >> 24), scale, bias));
    return r;
  }
};

template <>
struct WTile<MOE_I8_ROW> {
  u32x4_t v[4];  // [frag][half]; bytes hold code + 128
  __device__ __forceinline__ void load(const uint8_t* t, int lane) {
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = ((const u32x4_t*)t)[j * 64 + lane];
  }
  __device__ __forceinline__ u32x4_t frag(int f, int s) const {
    const u32x4_t& h = v[f * 2 + (s >> 1)];
    const uint32_t w0 = h[(s & 1) * 2], w1 = h[(s & 1) * 2 + 1];
    u32x4_t r;
    r[0] = pack_bf16x2((float)(w0 & 0xff) - 128.0f, (float)((w0 >> 8) & 0xff) - 128.0f);
    r[1] = pack_bf16x2((float)((w0 >> 16) & 0xff) - 128.0f, (float)(w0 >> 24) - 128.0f);
    r[2] = pack_bf16x2((float)(w1 & 0xff) - 128.0f, (float)((w1 >> 8) & 0xff) - 128.0f);
    r[3] = pack_bf16x2((float)((w1 >> 16) & 0xff) - 128.0f, (float)(w1 >> 24) - 128.0f);
    return r;
  }
};

// ---- one (row tile, column block) ----------------------------------------
struct TileJob {
  bool shared;
  int expert, start, cnt, nb;
};

struct Smem {
  uint16_t a[2][BM * 64];
  float wrow[BM];
  int src[BM];
};

template <int FMT, int STAGE>
__device__ __forceinline__ void run_tile(const FfnArgs& A, const TileJob& J, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Fw = J.shared ? A.Fs : A.F;
  const int K = STAGE == 1 ? A.d : Fw;
  const int nk = K / KC;
  const size_t tb = tile_bytes(FMT);
  const uint8_t* blob = J.shared ? A.shared_blob
                                 : A.routed_blob + (size_t)J.expert * expert_bytes(FMT, A.d, A.F);
  const size_t w1b = w1_bytes(FMT, A.d, Fw);
  const uint8_t* sect = STAGE == 1 ? blob : blob + w1b;
  const uint8_t* wt = sect + (size_t)(J.nb * WAVES + wave) * nk * tb;

  // rows of this tile: source row of the activations and folded router weight
  if (tid < BM) {
    const int m = tid;
    int src = -1;
    float wf = 0.0f;
    if (m < J.cnt) {
      if (STAGE == 1) {
        if (J.shared) {
          src = J.start + m;
          wf = 1.0f;
        } else {
          const int f = A.perm[J.start + m];
          src = f / A.k;
          wf = A.topk_w[f];
        }
      } else {
        src = J.start + m;
      }
    }
    sm.src[m] = src;
    sm.wrow[m] = wf;
  }
  __syncthreads();

  const uint16_t* abase = STAGE == 1 ? (const uint16_t*)A.hidden
                                     : (const uint16_t*)(J.shared ? A.h_shared : A.h_routed);
  const size_t astride = STAGE == 1 ? (size_t)A.d : (size_t)Fw;
  const int c8 = tid & 7;
  const uint16_t* arow[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int s = sm.src[(tid >> 3) + 32 * j];
    arow[j] = s >= 0 ? abase + (size_t)s * astride + c8 * 8 : nullptr;
  }
  const int nmf = (J.cnt + 31) >> 5;  // active 32-row fragments

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++) acc[i][0] = acc[i][1] = f32x16_t{};

  u32x4_t areg[4];
  auto load_a = [&](int kc) {
#pragma unroll
    for (int j = 0; j < 4; j++)
      areg[j] = arow[j] ? *(const u32x4_t*)(arow[j] + kc * KC) : u32x4_t{0, 0, 0, 0};
  };
  auto store_a = [&](uint16_t* dst) {
#pragma unroll
    for (int j = 0; j < 4; j++) *(u32x4_t*)(dst + lds_a_index((tid >> 3) + 32 * j, c8)) = areg[j];
  };
  auto compute = [&](const uint16_t* as, const WTile<FMT>& w) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const u32x4_t b0 = w.frag(0, s), b1 = w.frag(1, s);
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (i < nmf) {
          const u32x4_t av = *(const u32x4_t*)(as + lds_a_index(i * 32 + (lane & 31), ch));
          acc[i][0] = mfma32(av, b0, acc[i][0]);
          acc[i][1] = mfma32(av, b1, acc[i][1]);
        }
      }
    }
  };

  WTile<FMT> w0, w1;
  load_a(0);
  w0.load(wt, lane);
  store_a(sm.a[0]);
  __syncthreads();
  for (int kc = 0; kc < nk; kc += 2) {  // nk is even: K is a multiple of 128
    load_a(kc + 1);
    w1.load(wt + (size_t)(kc + 1) * tb, lane);
    compute(sm.a[0], w0);
    store_a(sm.a[1]);
    __syncthreads();
    if (kc + 2 < nk) {
      load_a(kc + 2);
      w0.load(wt + (size_t)(kc + 2) * tb, lane);
    }
    compute(sm.a[1], w1);
    if (kc + 2 < nk) store_a(sm.a[0]);
    __syncthreads();
  }

  // ---- epilogue
  const uint16_t* rscale =
      FMT == MOE_I8_ROW ? (const uint16_t*)(sect + (size_t)(STAGE == 1 ? (2 * Fw / 64) * (A.d / KC) : (A.d / 64) * (Fw / KC)) * tb)
                        : nullptr;
  if (STAGE == 1) {
    const int col = J.nb * H_COLS_BLOCK + wave * 32 + (lane & 31);
    float sg = 1.0f, su = 1.0f;
    if (FMT == MOE_I8_ROW) {
      sg = f16_bits_to_f32(rscale[col]);
      su = f16_bits_to_f32(rscale[Fw + col]);
    }
    uint16_t* hout = (uint16_t*)(J.shared ? A.h_shared : A.h_routed);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (i < nmf) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < J.cnt) {
            const float g = acc[i][0][r] * sg, u = acc[i][1][r] * su;
            const float h = sm.wrow[m] * silu_f(g) * u;
            hout[(size_t)(J.start + m) * Fw + col] = (uint16_t)(pack_bf16x2(h, 0.0f) & 0xffffu);
          }
        }
      }
    }
  } else {
    float* out = J.shared ? A.shared_out : A.out_assign;
#pragma unroll
    for (int f = 0; f < 2; f++) {
      const int col = J.nb * OUT_COLS_BLOCK + wave * 64 + f * 32 + (lane & 31);
      const float sc = FMT == MOE_I8_ROW ? f16_bits_to_f32(rscale[col]) : 1.0f;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (i < nmf) {
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int m = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m < J.cnt) out[(size_t)(J.start + m) * A.d + col] = acc[i][f][r] * sc;
          }
        }
      }
    }
  }
}

// Grid: slot-major with the column block fastest *within an XCD*: block b runs
// on XCD b % 8; slot = (b / (8*NB)) * 8 + b % 8, nb = (b / 8) % NB.  So all
// column blocks of one row tile share an XCD (and its L2 copy of the gathered
// activation rows), and empty slots spread evenly over the XCDs.
__device__ __forceinline__ bool decode_job(const FfnArgs& A, int NB, int ncols_routed,
                                           int ncols_shared, TileJob& J) {
  const int b = blockIdx.x;
  const int slot = (b / (8 * NB)) * 8 + (b & 7);
  J.nb = (b >> 3) % NB;
  if (slot < A.routed_slots) {
    if (slot >= *A.ntiles) return false;
    const int2 t = A.tiles[slot];
    J.shared = false;
    J.expert = t.x;
    J.start = A.offsets[t.x] + t.y;
    J.cnt = min(BM, A.offsets[t.x + 1] - J.start);
    return J.nb < ncols_routed;
  }
  const int s = slot - A.routed_slots;
  if (s >= A.shared_slots) return false;
  J.shared = true;
  J.expert = -1;
  J.start = s * BM;
  J.cnt = min(BM, A.T - J.start);
  return J.nb < ncols_shared;
}

template <int RF, int SF, int STAGE>
__global__ __launch_bounds__(256, 2) void ffn_kernel(FfnArgs A) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int NB = STAGE == 1 ? max(A.F, A.n_shared ? A.Fs : 0) / H_COLS_BLOCK : A.d / OUT_COLS_BLOCK;
  TileJob J;
  if (!decode_job(A, NB, STAGE == 1 ? A.F / H_COLS_BLOCK : NB,
                  STAGE == 1 ? A.Fs / H_COLS_BLOCK : NB, J))
    return;
  if (J.shared)
    run_tile<SF, STAGE>(A, J, sm);
  else
    run_tile<RF, STAGE>(A, J, sm);
}

template <int RF, int SF>
static hipError_t launch_pair(const FfnArgs& a, hipStream_t s) {
  const int slots = (a.routed_slots + a.shared_slots + 7) / 8 * 8;
  const int nb1 = max(a.F, a.n_shared ? a.Fs : 0) / H_COLS_BLOCK;
  const int nb2 = a.d / OUT_COLS_BLOCK;
  ffn_kernel<RF, SF, 1><<<slots * nb1, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_kernel<RF, SF, 2><<<slots * nb2, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ffn_bf16(const FfnArgs& a, hipStream_t s) {
  const int sf = a.n_shared ? a.shared_fmt : MOE_BF16;
  if (a.routed_fmt == MOE_BF16 && sf == MOE_BF16) return launch_pair<MOE_BF16, MOE_BF16>(a, s);
  if (a.routed_fmt == MOE_BF16 && sf == MOE_I8_ROW) return launch_pair<MOE_BF16, MOE_I8_ROW>(a, s);
  if (a.routed_fmt == MOE_I4_G32 && sf == MOE_BF16) return launch_pair<MOE_I4_G32, MOE_BF16>(a, s);
  if (a.routed_fmt == MOE_I4_G32 && sf == MOE_I8_ROW)
    return launch_pair<MOE_I4_G32, MOE_I8_ROW>(a, s);
  return hipErrorInvalidValue;
}

// ---- fp32 path: plain fp32 FMAs on canonical row-major weights --------------
// Block = one row tile x 64 columns, one thread per column, rows in sequence.
__global__ __launch_bounds__(64) void ffn_f32_stage1(FfnArgs A, int NB) {
  TileJob J;
  if (!decode_job(A, NB, A.F / 64, A.n_shared ? A.Fs / 64 : 0, J)) return;
  const int Fw = J.shared ? A.Fs : A.F;
  const int j = J.nb * 64 + threadIdx.x;
  const float* blob = (const float*)(J.shared ? A.shared_blob
                                              : A.routed_blob + (size_t)J.expert * expert_bytes(MOE_F32, A.d, A.F));
  const float* wg = blob + (size_t)j * A.d;
  const float* wu = blob + (size_t)(Fw + j) * A.d;
  float* hout = (float*)(J.shared ? A.h_shared : A.h_routed);
  const float* X = (const float*)A.hidden;
  for (int m = 0; m < J.cnt; m++) {
    int t;
    float wf;
    if (J.shared) {
      t = J.start + m;
      wf = 1.0f;
    } else {
      const int f = A.perm[J.start + m];
      t = f / A.k;
      wf = A.topk_w[f];
    }
    const float* x = X + (size_t)t * A.d;
    float g = 0.0f, u = 0.0f;
    for (int i = 0; i < A.d; i++) {
      g = fmaf(wg[i], x[i], g);
      u = fmaf(wu[i], x[i], u);
    }
    hout[(size_t)(J.start + m) * Fw + j] = wf * (g / (1.0f + expf(-g))) * u;
  }
}

__global__ __launch_bounds__(64) void ffn_f32_stage2(FfnArgs A, int NB) {
  TileJob J;
  if (!decode_job(A, NB, NB, NB, J)) return;
  const int Fw = J.shared ? A.Fs : A.F;
  const int n = J.nb * 64 + threadIdx.x;
  const float* blob = (const float*)(J.shared ? A.shared_blob
                                              : A.routed_blob + (size_t)J.expert * expert_bytes(MOE_F32, A.d, A.F));
  const float* wd = blob + (size_t)2 * Fw * A.d + (size_t)n * Fw;
  const float* H = (const float*)(J.shared ? A.h_shared : A.h_routed);
  float* out = J.shared ? A.shared_out : A.out_assign;
  for (int m = 0; m < J.cnt; m++) {
    const float* h = H + (size_t)(J.start + m) * Fw;
    float o = 0.0f;
    for (int j = 0; j < Fw; j++) o = fmaf(wd[j], h[j], o);
    out[(size_t)(J.start + m) * A.d + n] = o;
  }
}

hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s) {
  const int slots = (a.routed_slots + a.shared_slots + 7) / 8 * 8;
  const int nb1 = max(a.F, a.n_shared ? a.Fs : 0) / 64, nb2 = a.d / 64;
  ffn_f32_stage1<<<slots * nb1, 64, 0, s>>>(a, nb1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_f32_stage2<<<slots * nb2, 64, 0, s>>>(a, nb2);
  return hipGetLastError();
}

}  // namespace moe
