// ffn_mx.hip -- expert-grouped SwiGLU GEMMs of MXFP4 W4A4 routed experts
// ("anvil-serving" dossier, Qwen3.8-Flash-Next entry, section "Quantization
// boundary": 4-bit weights and activations on the routed experts, the shared
// expert 16-bit), in the OCP Microscaling FP4 format that CDNA4's scaled
// MFMA (16x16x128, e2m1 operands, one E8M0 scale per 32 K per row) consumes.
//
//   x_to_mx_kernel   x -> e2m1 codes + E8M0 scales, block by block of 32
//                    (OCP MX rule), one row per token, into the workspace
//   ffn_mx_kernel<1> routed tiles: g, u = Wg xq, Wu xq on the FP4 MFMA;
//                    h = w * silu(g) * u in fp32, quantized per row and 32 h
//                    columns (one wave's columns) -> hq, hsc
//   ffn_mx_kernel<2> routed tiles: out_assign = Wd hq on the FP4 MFMA
// Shared-expert tiles of the same launches run the 16-bit path of
// ffn_kernels.h on the unquantized bf16 x.
//
// Work unit and grid as in ffn_kernels.h (row tile of up to 16 * MAXMF rows x
// one column block of 4 waves; each wave one run of 64 weight rows).  A K
// chunk is 128: per chunk a wave reads one 4352-byte weight tile (4 fragments
// x 16 bytes of codes + one scale dword per lane) straight into registers,
// and the block stages the tile rows' codes (64 bytes a row) and scales
// through LDS, double-buffered.  No dequantization: codes and scales feed the
// MFMA as they are.
//
// Activation layout, chunk-major (x's codes: n = T rows in token order, which
// the gate/up tiles gather through perm while staging; h's codes: n = T*k
// rows in route-plan order, so the rows of a down tile are contiguous) --
//   codes   q[(kc * n + p) * 64 + kb * 16 + j]   chunk kc, row p, 32-K block kb
//   scales  s[((kc / 2) * n + p) * 8 + (kc % 2) * 4 + kb]   (pairs of chunks)
// The gate/up epilogue of column block nb writes chunk nb of h (its 128 h
// columns) whole.
#include <utility>

#include "ffn_kernels.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, Is...>) {
  (fn(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  static_for_impl(fn, std::make_integer_sequence<int, N>{});
}

// acc += A (16 rows x 128 K) * B (16 columns x 128 K)^T, e2m1 operands.  Lane
// l supplies row / column l % 16 and K block l / 16 (32 codes, element 2j in
// the low nibble of byte j); byte OA of sa is the E8M0 scale of its A block,
// byte OB of sb that of its B block.  The result layout is the 16x16x32 one.
template <int OA, int OB>
__device__ __forceinline__ f32x4_t mfma_fp4(const u32x4_t& a, uint32_t sa, const u32x4_t& b,
                                            uint32_t sb, f32x4_t c) {
  const i32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, OA, (int)sa, OB,
                                                          (int)sb);
}

// Two fp32 values, already divided by their block scale, to two e2m1 codes
// (nearest, ties to even, saturated at +-6) in byte SEL of `old` (the first
// value in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Shared exponent of an MX block from the bits of its largest magnitude:
// floor(log2 amax) - 2, clamped to [-127, 127] (-127 for zero and subnormal
// maxima).  Returns E; *inv = 2^-E (a normal float for every such E).
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits, float* inv) {
  const int E = max((int)(amax_bits >> 23) - 129, -127);
  *inv = __uint_as_float((uint32_t)(127 - E) << 23);
  return E;
}

// ---- x -> MXFP4 --------------------------------------------------------------
// One thread per 32-element block: thread g takes block kb = g % 4 of chunk kc
// of token t ((g / 4) = kc * n + t, n = T), so four threads read 256
// contiguous bytes of the token's row and write one row's 64 code bytes, and
// successive rows follow each other in the output.  Each token is quantized
// once; its k assignments' tiles gather its codes.
__global__ __launch_bounds__(256) void x_to_mx_kernel(int n, int d, const uint16_t* __restrict__ x,
                                                      uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xsc) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nblk = (int64_t)n * (d / 32);
  if (g >= nblk) return;
  const int kb = (int)(g & 3);
  const int64_t cp = g >> 2;  // kc * n + t
  const int kc = (int)(cp / n);
  const int64_t t = cp - (int64_t)kc * n;
  const int p = (int)t;
  const u32x4_t* src = (const u32x4_t*)(x + t * d + (kc * 4 + kb) * 32);
  u32x4_t v[4];
#pragma unroll
  for (int j = 0; j < 4; j++) v[j] = src[j];
  uint32_t m = 0;  // largest |x| as float bits
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int w = 0; w < 4; w++) m = max(m, max((v[j][w] << 16) & 0x7fffffffu, v[j][w] & 0x7fff0000u));
  float inv;
  const int E = mx_exponent(m, &inv);
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    // dword w of piece j holds elements 8j + 2w (low half) and 8j + 2w + 1
    uint32_t c = 0;
    c = cvt_fp4x2<0>(c, bf16_lo(v[j][0]) * inv, bf16_hi(v[j][0]) * inv);
    c = cvt_fp4x2<1>(c, bf16_lo(v[j][1]) * inv, bf16_hi(v[j][1]) * inv);
    c = cvt_fp4x2<2>(c, bf16_lo(v[j][2]) * inv, bf16_hi(v[j][2]) * inv);
    c = cvt_fp4x2<3>(c, bf16_lo(v[j][3]) * inv, bf16_hi(v[j][3]) * inv);
    o[j] = c;
  }
  *(u32x4_t*)(xq + cp * 64 + kb * 16) = o;
  xsc[((int64_t)(kc >> 1) * n + p) * 8 + (kc & 1) * 4 + kb] = (uint8_t)(E + 127);
}

// ---- weight registers of one MXFP4 wave tile (64 rows x 128 K) -------------
struct WTileMx {
  u32x4_t v[4];  // fragment f: the lane's 32 codes (row l % 16, K block l / 16)
  uint32_t sc;   // byte f: the E8M0 scale of fragment f's row and block
  template <bool NT>
  __device__ __forceinline__ void load(const uint8_t* t, int lane) {
#pragma unroll
    for (int f = 0; f < 4; f++) v[f] = ldw<NT>(t + f * 1024, lane);
    const uint32_t* sp = (const uint32_t*)(t + 4096) + lane;
    sc = NT ? __builtin_nontemporal_load(sp) : *sp;
  }
};

// Activation rows of one 128-K chunk in LDS: 64 code bytes a row as four
// 16-byte pieces, piece kb of row r at slot kb ^ swz(r), so the pieces that 8
// (or 16) consecutive rows read at one kb, and that 16 consecutive pieces
// write, fall in distinct 16-byte bank groups.  The scales sit apart as
// [kb][r % 16][r / 16] bytes: a lane reads the scales of all its row
// fragments with one 8-byte load.
__device__ __forceinline__ int mx_lds_index(int row, int kb) {
  const int swz = ((row >> 1) & 3) ^ ((row >> 3) & 1);
  return row * 64 + ((kb ^ swz) << 4);
}

template <int MAXMF>
struct SmemMx {
  uint8_t a[2][MAXMF * 16 * 64];
  uint8_t s[2][4 * 16 * 8];
  float wrow[MAXMF * 16];
  int src[MAXMF * 16];  // A row of each tile row (gate/up: its token)
};

// Stage-1 epilogue: h = w * silu(g) * u of the wave's 32 h columns, quantized
// to MXFP4 per row (the 32 columns are one block).  Row i*16 + 4*(lane/16) + r
// of the tile holds, in lane l, column 16 f + l % 16 for f = 0, 1 (gate
// fragments f, up fragments f + 2).  The row maximum runs over the 16 lanes of
// a DPP row; lanes l and l^1 then trade their codes so each lane holds whole
// bytes (two columns) of two rows.  The block's codes (64 bytes a row: 16 per
// wave) and scales (4 bytes a row) are gathered in LDS (`hl`, `sl`, free after
// the K loop) and leave as one 16-byte store per row piece and one 4-byte
// store per row, into chunk nb of the plan-order chunk-major layout.
template <int NMF, typename RowW>
__device__ __forceinline__ void store_h_mx(const FfnArgs& A, int start, int cnt, int nb,
                                           const f32x4_t (&acc)[NMF][4], RowW wrow, uint8_t* hl,
                                           uint8_t* sl) {
  constexpr int ROWS = NMF * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, quad = 4 * (lane >> 4);
  const bool odd = lane & 1;
  __syncthreads();  // every wave is done reading the staging buffers
#pragma unroll
  for (int i = 0; i < NMF; i++) {
    float h0[4], h1[4];
    uint32_t eb[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float w = wrow(i, r);
      h0[r] = w * silu_fast(acc[i][0][r]) * acc[i][2][r];
      h1[r] = w * silu_fast(acc[i][1][r]) * acc[i][3][r];
      uint32_t m = max(__float_as_uint(h0[r]) & 0x7fffffffu, __float_as_uint(h1[r]) & 0x7fffffffu);
      // max over the 16 lanes of the DPP row: quad_perm [1,0,3,2], [2,3,0,1],
      // then row_half_mirror and row_mirror
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, false));
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x140, 0xF, 0xF, false));
      float inv;
      eb[r] = (uint32_t)(mx_exponent(m, &inv) + 127);
      h0[r] *= inv;
      h1[r] *= inv;
    }
    // nibble 4 f + r = the code of (row r, fragment f)
    uint32_t code = 0;
    code = cvt_fp4x2<0>(code, h0[0], h0[1]);
    code = cvt_fp4x2<1>(code, h0[2], h0[3]);
    code = cvt_fp4x2<2>(code, h1[0], h1[1]);
    code = cvt_fp4x2<3>(code, h1[2], h1[3]);
    const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)code, 0xB1, 0xF, 0xF, false);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int r = odd ? 2 + q : q;  // the even lane takes rows 0, 1, the odd lane 2, 3
      const int row = i * 16 + quad + r;
#pragma unroll
      for (int f = 0; f < 2; f++) {
        const int n = 4 * (4 * f + r);
        const uint32_t mine = (code >> n) & 15u, oth = (other >> n) & 15u;
        hl[row * 64 + wave * 16 + 8 * f + (c >> 1)] =
            (uint8_t)(odd ? (oth | (mine << 4)) : (mine | (oth << 4)));
      }
    }
    if (c < 4) sl[(i * 16 + quad + c) * 4 + wave] = (uint8_t)(c == 0 ? eb[0] : c == 1 ? eb[1] : c == 2 ? eb[2] : eb[3]);
  }
  __syncthreads();
  // chunk nb of h: the tile's rows are contiguous (plan-order chunk-major)
  const size_t n = (size_t)A.T * A.k;
  uint8_t* hq = A.hq + ((size_t)nb * n + start) * 64;
#pragma unroll
  for (int q = tid; q < ROWS * 4; q += WAVES * 64)
    if ((q >> 2) < cnt) *(u32x4_t*)(hq + q * 16) = *(const u32x4_t*)(hl + q * 16);
  if (tid < ROWS && tid < cnt)
    *(uint32_t*)(A.hsc + ((size_t)(nb >> 1) * n + start + tid) * 8 + (nb & 1) * 4) =
        *(const uint32_t*)(sl + tid * 4);
}

// One routed (row tile, column block) of an MXFP4 layer.
template <int STAGE, int MAXMF, int PF, bool NT>
__device__ __forceinline__ void run_tile_mx(const FfnArgs& A, const TileJob& J, SmemMx<MAXMF>& sm) {
  constexpr int NMF = MAXMF;
  constexpr int ROWS = MAXMF * 16;
  constexpr int PIECES = ROWS * 4;  // 16-byte code pieces of one chunk
  constexpr int PPT = (PIECES + WAVES * 64 - 1) / (WAVES * 64);
  static_assert(PPT <= 2, "code staging holds at most 2 pieces per thread");
  static_assert(MAXMF > 2 || PPT == 1, "small tiles stage one piece per thread");
  static_assert(PF == 2, "the scale pairs below assume a lead of two chunks");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = STAGE == 1 ? A.d : A.F;
  const int nk = K / KC_MX;
  const int run = J.nb * WAVES + wave;
  const uint8_t* blob = A.routed_blob + (size_t)J.expert * expert_bytes(MOE_MXFP4, A.d, A.F);
  const uint8_t* sect = STAGE == 1 ? blob : blob + w1_bytes(MOE_MXFP4, A.d, A.F);
  const uint8_t* wnext = sect + (size_t)run * nk * TILE_BYTES_MX4;

  // Tile row m: folded router weight and A row (gate/up: token perm / k of
  // x's codes; down: plan row start + m of h's).  Rows past the tile's end
  // read the tile's first row (never stored).
  for (int m = tid; m < ROWS; m += WAVES * 64) {
    const int mm = m < J.cnt ? m : 0;
    if (STAGE == 1) {
      const int f = A.perm[J.start + mm];
      sm.wrow[m] = m < J.cnt ? A.topk_w[f] : 0.0f;
      sm.src[m] = f / A.k;
    } else {
      sm.wrow[m] = 0.0f;
      sm.src[m] = J.start + mm;
    }
  }
  __syncthreads();

  // chunk-major rows: one chunk of codes, one chunk pair of scales apart
  const size_t n = STAGE == 1 ? (size_t)A.T : (size_t)A.T * A.k;
  const size_t qstep = n * 64, sstep = n * 8;
  const uint8_t* qbase = STAGE == 1 ? A.xq : A.hq;
  const uint8_t* sbase = STAGE == 1 ? A.xsc : A.hsc;
  const uint8_t* aq[PPT];
  int aq_lds[PPT];
#pragma unroll
  for (int j = 0; j < PPT; j++) {
    const int q = (tid + WAVES * 64 * j) % PIECES;  // piece q: row q / 4, K block q % 4
    const int r = q >> 2, kb = q & 3;
    aq[j] = qbase + (size_t)sm.src[r] * 64 + kb * 16;
    aq_lds[j] = mx_lds_index(r, kb);
  }
  // scales: thread tid stages row tid % ROWS (4 bytes a chunk)
  const int srow = tid % ROWS;
  const uint8_t* as = sbase + (size_t)sm.src[srow] * 8;
  const int s_lds = (srow & 15) * 8 + (srow >> 4);  // + kb * 128

  f32x4_t acc[NMF][4];
#pragma unroll
  for (int i = 0; i < NMF; i++)
#pragma unroll
    for (int f = 0; f < 4; f++) acc[i][f] = f32x4_t{0, 0, 0, 0};

  // Ring slot p holds chunk kc with kc % 2 == p.  The scales of an even chunk
  // and the next one arrive together in `apair` (one 8-byte load per row
  // every two chunks).
  u32x4_t areg[PF][PPT];
  uint2 apair;
  // Small tiles have fewer pieces than threads: only the threads that own a
  // distinct piece (whole waves) load and stage it.  Large tiles let every
  // thread load (some pieces twice, same bytes to the same place): measured,
  // the predicated form is much slower there.
  constexpr bool PRED = MAXMF <= 2;
  const bool own0 = !PRED || tid < PIECES, own_s = !PRED || tid < ROWS;
  auto load_a = [&](int kc, int p) {
#pragma unroll
    for (int j = 0; j < PPT; j++)
      if (own0) areg[p][j] = *(const u32x4_t*)(aq[j] + (size_t)kc * qstep);
    if (p == 0 && own_s) apair = *(const uint2*)(as + (size_t)(kc >> 1) * sstep);
  };
  auto store_a = [&](int buf, int p, uint32_t sc) {
#pragma unroll
    for (int j = 0; j < PPT; j++)
      if (own0) *(u32x4_t*)(sm.a[buf] + aq_lds[j]) = areg[p][j];
    if (own_s) {
#pragma unroll
      for (int kb = 0; kb < 4; kb++) sm.s[buf][kb * 128 + s_lds] = (uint8_t)(sc >> (8 * kb));
    }
  };
  const int am = lane & 15, akb = lane >> 4;
  auto compute = [&](int buf, const WTileMx& w) {
    u32x4_t av[NMF];
#pragma unroll
    for (int i = 0; i < NMF; i++) av[i] = *(const u32x4_t*)(sm.a[buf] + mx_lds_index(i * 16 + am, akb));
    uint32_t sa[2];
    if constexpr (NMF > 4) {
      const uint2 t = *(const uint2*)(sm.s[buf] + akb * 128 + am * 8);
      sa[0] = t.x;
      sa[1] = t.y;
    } else {
      sa[0] = *(const uint32_t*)(sm.s[buf] + akb * 128 + am * 8);
      sa[1] = 0;
    }
    static_for<4>([&](auto F) {
      constexpr int f = decltype(F)::value;
      static_for<NMF>([&](auto I) {
        constexpr int i = decltype(I)::value;
        acc[i][f] = mfma_fp4<i & 3, f>(av[i], sa[i >> 2], w.v[f], w.sc, acc[i][f]);
      });
    });
  };

  // The peeled pipeline of ffn_kernels.h's tile_body with a lead of two
  // chunks: step kc issues the activation and weight loads of chunk kc + 2 in
  // the order they are waited for; nk is even (the ABI's width checks).
  WTileMx ring[PF];
#pragma unroll
  for (int p = 0; p < PF; p++) {
    load_a(p, p);
    ring[p].template load<NT>(wnext, lane);
    wnext += TILE_BYTES_MX4;
  }
  store_a(0, 0, apair.x);
  __syncthreads();
  for (int kc0 = 0; kc0 < nk - PF; kc0 += PF) {
    // step 0: chunk kc0 from LDS; loads of chunk kc0 + 2 (and the scale pair
    // of kc0 + 2, kc0 + 3); stages chunk kc0 + 1, whose scale is the odd half
    // of the pair being replaced
    const uint32_t s_odd = apair.y;
    load_a(kc0 + 2, 0);
    compute(0, ring[0]);
    ring[0].template load<NT>(wnext, lane);
    wnext += TILE_BYTES_MX4;
    store_a(1, 1, s_odd);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // step 1: chunk kc0 + 1; loads of chunk kc0 + 3; stages chunk kc0 + 2
    load_a(kc0 + 3, 1);
    compute(1, ring[1]);
    ring[1].template load<NT>(wnext, lane);
    wnext += TILE_BYTES_MX4;
    store_a(0, 0, apair.x);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  compute(0, ring[0]);  // the last two chunks: nothing more to load
  store_a(1, 1, apair.y);
  __syncthreads();
  compute(1, ring[1]);

  const int quad = 4 * (lane >> 4);
  auto wrow = [&](int i, int r) { return sm.wrow[i * 16 + quad + r]; };
  if constexpr (STAGE == 1) {
    store_h_mx<NMF>(A, J.start, J.cnt, J.nb, acc, wrow, sm.a[0], sm.s[0]);
  } else {
    store_wave_tile<MOE_MXFP4, 2, NMF, false>(A, false, J.start, J.cnt, run, A.F, sect, acc, wrow,
                                               [](int, int) { return 1.0f; });
  }
}

// Routed tiles of a 96-row kernel with fewer rows run a body with fewer row
// fragments (as run_routed_tile in ffn_kernels.h; measured -1% at T=4096).
template <int STAGE, int MAXMF, int PF, bool NT>
__device__ __forceinline__ void run_routed_tile_mx(const FfnArgs& A, const TileJob& J,
                                                   SmemMx<MAXMF>& sm) {
  if constexpr (MAXMF == 6) {
    if (J.cnt <= 32)
      return run_tile_mx<STAGE, 2, PF, NT>(A, J, *reinterpret_cast<SmemMx<2>*>(&sm));
    if (J.cnt <= 64)
      return run_tile_mx<STAGE, 4, PF, NT>(A, J, *reinterpret_cast<SmemMx<4>*>(&sm));
    if (J.cnt <= 80)
      return run_tile_mx<STAGE, 5, PF, NT>(A, J, *reinterpret_cast<SmemMx<5>*>(&sm));
  }
  run_tile_mx<STAGE, MAXMF, PF, NT>(A, J, sm);
}

template <int SF, int STAGE, int MAXMF, int PF>
__global__ __launch_bounds__(WAVES * 64, 8 / WAVES) void ffn_mx_kernel(FfnArgs A) {
  __shared__ __attribute__((aligned(16))) union {
    Smem<MAXMF> b;
    SmemMx<MAXMF> m;
  } sm;
  const int nr = STAGE == 1 ? col_blocks(A.F / H_COLS_WAVE) : col_blocks(A.d / OUT_COLS_WAVE);
  const int ns = STAGE == 1 ? (A.n_shared ? col_blocks(A.Fs / H_COLS_WAVE) : 0) : nr;
  TileJob J;
  if (!decode_job<true>(A, max(nr, ns), nr, ns, MAXMF * 16, J)) return;
  // Routed weights stream past the caches at every call size (measured: at
  // T=4096 the few experts whose rows span two tiles re-read theirs, and
  // still the layer is faster than with cacheable loads).
  constexpr bool NT_ROUTED = true;
  if (J.shared)
    run_tile<SF, STAGE, MAXMF, LEAD_I4, false, false>(A, J, sm.b);
  else
    run_routed_tile_mx<STAGE, MAXMF, PF, NT_ROUTED>(A, J, sm.m);
}

template <int SF, int MAXMF>
static hipError_t launch_mx_stages(const FfnArgs& a0, hipStream_t s) {
  FfnArgs a = a0;
  a.shared_slots = a.n_shared ? (a.T + MAXMF * 16 - 1) / (MAXMF * 16) : 0;
  const int slots = (a.routed_slots + a.shared_slots + 7) / 8 * 8;
  const int nb1 = col_blocks(max(a.F, a.n_shared ? a.Fs : 0) / H_COLS_WAVE);
  const int nb2 = col_blocks(a.d / OUT_COLS_WAVE);
  const int64_t blocks = (int64_t)a.T * (a.d / 32);
  x_to_mx_kernel<<<(unsigned)((blocks + 255) / 256), 256, 0, s>>>(
      a.T, a.d, (const uint16_t*)a.hidden, a.xq, a.xsc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_mx_kernel<SF, 1, MAXMF, LEAD_MX><<<slots * nb1, WAVES * 64, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_mx_kernel<SF, 2, MAXMF, LEAD_MX><<<slots * nb2, WAVES * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int SF>
static hipError_t launch_mx_sf(const FfnArgs& a, hipStream_t s) {
  if (a.T <= 16) return launch_mx_stages<SF, 1>(a, s);
  if (a.T <= 32) return launch_mx_stages<SF, 2>(a, s);
  return launch_mx_stages<SF, BM / 16>(a, s);
}

hipError_t launch_ffn_mx(const FfnArgs& a, hipStream_t s) {
  const int sf = a.n_shared ? a.shared_fmt : MOE_BF16;
  if (sf == MOE_BF16) return launch_mx_sf<MOE_BF16>(a, s);
  if (sf == MOE_I8_ROW) return launch_mx_sf<MOE_I8_ROW>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
