// ffn_kernels.h -- expert-grouped SwiGLU GEMMs ("Qwen3.8-Flash-Next-Dual-GPU"
// README, section "Dedicated prefill lane", steps 2-4).
//
// Work unit: one row tile (up to BM = 96 consecutive rows of one expert's group
// in the route plan, or up to 96 tokens of the always-active shared expert)
// times one column block.  A block is 4 wave64s:
//   stage 1: h[p] = w_p * silu(Wg x_t) (.) (Wu x_t)   -> h (bf16), rows p
//            each wave owns 32 h columns: 32 gate rows and 32 up rows of W1
//   stage 2: out[p] = Wd h[p]                          -> fp32, one row per
//            assignment (out_assign) or per token (shared_out)
//            each wave owns 64 output columns
// Activations (x rows gathered through perm, or h rows) are staged through
// LDS, 64 K at a time, double-buffered, and read as MFMA A operands by all 4
// waves.  Weights stream straight from HBM into each wave's registers in the
// tile order moe_pack_experts wrote them (one contiguous run per wave), PF
// chunks ahead, and are dequantized in registers: to fp16 for the gate/up
// products of int4 and b-bit layers (which run fp16 MFMA on an fp16 copy of
// x), to bf16 otherwise (codes times the fp16 group scale, rounded to nearest
// even; int8 codes enter exactly and their row scale multiplies the fp32
// accumulator); MFMA 16x16x32 with fp32 accumulation.  A wave covers all rows
// of its tile, so each weight is read and dequantized once per row tile.  A
// tile runs a body built for just enough 16-row fragments (run_routed_tile);
// fragments past its last row compute copies of its first row and are never
// stored.
#pragma once

#include "wave_tile.h"

namespace moe {

// ---- one (row tile, column block) ----------------------------------------
struct TileJob {
  bool shared;
  int expert, start, cnt, nb;
};

// SLOTS: A chunks held in LDS -- 4 for tiles with a 4-chunk load lead (two
// chunks are read while the next two are written, one barrier per two
// chunks), 2 otherwise.
template <int MAXMF, int SLOTS = 2>
struct Smem {
  uint16_t a[SLOTS][MAXMF * 16 * 64];
  float wrow[MAXMF * 16];
  float xs[MAXMF * 16];  // power of two to undo on fp16-staged rows
  int src[MAXMF * 16];
};

// Per-tile constants shared by the setup and the main loop.
struct TileCtx {
  int Fw, nk;
  int run;              // this wave's run of 64 weight rows
  const uint8_t* sect;  // W1 or W2 section of this expert's blob
  const uint8_t* wt;    // this wave's run of weight tiles
  const uint8_t* abase; // activation rows (x, its fp16 copy, or h)
  uint32_t aoff[3];     // byte offset of each staged piece's row and 16 bytes
};

// Lead of the loads, in K chunks: 4 for int4 and 2-bit codes (the bytes of the
// call); 2 for bf16 tiles (4x the bytes and registers of an int4 tile), int8
// shared tiles (re-read from cache by every row tile) and the 3- and 5- to
// 8-bit codes (their registers).
template <int FMT, int PF_MAX>
constexpr int slots_of() { return lead_of(FMT, PF_MAX) == 4 ? 4 : 2; }

template <int FMT, int STAGE, int MAXMF, int PF_MAX, bool F16, bool NT>
__device__ __forceinline__ void tile_body(const FfnArgs& A, const TileJob& J,
                                          Smem<MAXMF, slots_of<FMT, PF_MAX>()>& sm,
                                          const TileCtx& C,
                                          WTile<FMT> (&ring)[lead_of(FMT, PF_MAX)]) {
  constexpr int NMF = MAXMF;
  constexpr int PF = lead_of(FMT, PF_MAX);
  constexpr int ROWS = MAXMF * 16;
  constexpr int PIECES = ROWS * 8;  // 16-byte pieces of one A chunk
  constexpr int PPT = (PIECES + WAVES * 64 - 1) / (WAVES * 64);
  const int tid = threadIdx.x, lane = tid & 63;
  const int nk = C.nk;
  const size_t tb = tile_bytes(FMT);

  f32x4_t acc[NMF][4];
#pragma unroll
  for (int i = 0; i < NMF; i++)
#pragma unroll
    for (int f = 0; f < 4; f++) acc[i][f] = f32x4_t{0, 0, 0, 0};

  // Chunk c of the activations travels in register set c % PF, then lands in
  // LDS buffer c & 1; chunk c of the weights sits in ring slot c % PF.
  u32x4_t areg[PF][PPT];
  const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(C.abase);
  auto load_a = [&](int kc, u32x4_t (&dst)[PPT]) {
    const BufSrc src{arsrc, (uint32_t)(kc * KC * 2)};
#pragma unroll
    for (int j = 0; j < PPT; j++) dst[j] = src.ld16<false>(C.aoff[j]);
  };
  // Thread tid stages pieces (tid + 256 j) mod PIECES: in small tiles some
  // pieces are stored twice (same bytes, same place), so no store sits
  // behind a branch.
  auto store_a = [&](uint16_t* dst, const u32x4_t (&src)[PPT]) {
#pragma unroll
    for (int j = 0; j < PPT; j++) {
      const int q = (tid + WAVES * 64 * j) % PIECES;
      *(u32x4_t*)(dst + lds_a_index(q >> 3, q & 7)) = src[j];
    }
  };
  const F16Consts f16k = {0x000f000fu, 0x00f000f0u, 0x64006400u, 0x54005400u};
  // One chunk on all MAXMF row fragments.  Fragments past the tile's last row
  // hold copies of its first row and are never stored: a straight-line run of
  // MFMAs with no branch beats skipping them (a scalar branch per fragment
  // breaks the MFMA issue stream).
  auto compute = [&](const uint16_t* as, const WTile<FMT>& w) {
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int ch = 4 * s + (lane >> 4);
      u32x4_t av[NMF];
#pragma unroll
      for (int i = 0; i < NMF; i++)
        av[i] = *(const u32x4_t*)(as + lds_a_index(i * 16 + (lane & 15), ch));
#pragma unroll
      for (int f = 0; f < 4; f++) {
        const u32x4_t b = F16 ? w.frag16(f, s, f16k) : w.frag(f, s, f16k);
#pragma unroll
        for (int i = 0; i < NMF; i++)
          acc[i][f] = F16 ? mfma16x16_f16(av[i], b, acc[i][f]) : mfma16x16(av[i], b, acc[i][f]);
      }
    }
  };

  // The loop is peeled so that no load sits behind a condition: step kc
  // issues the activation and weight loads of chunk kc + PF, in the order
  // they will be waited for.  The memory counter retires loads in issue
  // order, so a wait then covers the chunk it needs and nothing issued after
  // it, and PF chunks stay in flight.  nk is a multiple of PF (the ABI's width
  // checks).
  static_assert(PF == 2 || PF == 4, "load lead must be 2 or 4 chunks");
  // stage 1: the caller issued the first PF weight chunks
  BufSrc wnext{buffer_rsrc(C.wt), (uint32_t)(STAGE == 1 ? PF * tb : 0)};
#pragma unroll
  for (int p = 0; p < PF; p++) {
    load_a(p, areg[p]);
    if constexpr (STAGE != 1) {
      ring[p].template load<NT>(wnext, lane);
      wnext.soff += (uint32_t)tb;
    }
  }
  if constexpr (PF == 4) {
    // Four LDS slots: step c computes chunk c from slot c % 4 and stores
    // chunk c + 2 into slot (c + 2) % 4, whose chunk c - 2 every wave read
    // before the last barrier; a barrier after every second step publishes
    // the two chunks stored since the previous one.  A chunk's activations
    // wait two steps in registers between load and store.
    store_a(sm.a[0], areg[0]);
    store_a(sm.a[1], areg[1]);
    __syncthreads();
    for (int kc0 = 0; kc0 < nk - PF; kc0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; p++) {
        load_a(kc0 + p + PF, areg[p]);  // set p held chunk kc0 + p, stored two steps ago
        if constexpr (MAXMF <= 2) __builtin_amdgcn_s_setprio(1);
        compute(sm.a[p], ring[p]);
        if constexpr (MAXMF <= 2) __builtin_amdgcn_s_setprio(0);
        ring[p].template load<NT>(wnext, lane);
        wnext.soff += (uint32_t)tb;
        store_a(sm.a[(p + 2) % 4], areg[(p + 2) % PF]);
        if (p & 1) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int p = 0; p < PF; p++) {  // the last PF chunks: nothing more to load
      compute(sm.a[p], ring[p]);
      if (p < 2) store_a(sm.a[p + 2], areg[p + 2]);
      if (p == 1) __syncthreads();
    }
  } else {
  store_a(sm.a[0], areg[0]);
  __syncthreads();
  for (int kc0 = 0; kc0 < nk - PF; kc0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; p++) {
      load_a(kc0 + p + PF, areg[p]);  // set p held chunk kc0 + p, already in LDS
      // Small tiles raise the wave's issue priority over its dequantization
      // and MFMAs, so a wave with a chunk ready runs it ahead of the block's
      // other waves, which are waiting on loads (T=32 graph -3.5%; no gain at
      // 96-row tiles: T=4096 +0.7%).
      if constexpr (MAXMF <= 2) __builtin_amdgcn_s_setprio(1);
      compute(sm.a[p & 1], ring[p]);
      if constexpr (MAXMF <= 2) __builtin_amdgcn_s_setprio(0);
      ring[p].template load<NT>(wnext, lane);
      wnext.soff += (uint32_t)tb;
      store_a(sm.a[(p + 1) & 1], areg[(p + 1) % PF]);
      __syncthreads();
      // keep the scheduler from hoisting the next chunk's dequantization
      // into this one (it would hold two chunks' registers at once)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int p = 0; p < PF; p++) {  // the last PF chunks: nothing more to load
    compute(sm.a[p & 1], ring[p]);
    if (p + 1 < PF) {
      store_a(sm.a[(p + 1) & 1], areg[p + 1]);
      __syncthreads();
    }
  }
  }

  const int quad = 4 * (lane >> 4);
  store_wave_tile<FMT, STAGE, NMF, F16>(
      A, J.shared, J.start, J.cnt, C.run, C.Fw, C.sect, acc,
      [&](int i, int r) { return sm.wrow[i * 16 + quad + r]; },
      [&](int i, int r) { return sm.xs[i * 16 + quad + r]; });
}

// F16: stage-1 tile on fp16 MFMA, A rows from the fp16 copy of the
// activations (scaled per token by a power of two, undone in the epilogue).
template <int FMT, int STAGE, int MAXMF, int PF_MAX, bool F16, bool NT>
__device__ __forceinline__ void run_tile(const FfnArgs& A, const TileJob& J,
                                         Smem<MAXMF, slots_of<FMT, PF_MAX>()>& sm) {
  constexpr int ROWS = MAXMF * 16;
  constexpr int PIECES = ROWS * 8;  // 16-byte pieces of one A chunk
  constexpr int PPT = (PIECES + WAVES * 64 - 1) / (WAVES * 64);
  static_assert(PPT <= 3, "A staging holds at most 3 pieces per thread");
  // the wave index as a scalar: every weight address of the wave is then
  // uniform (a scalar base plus the lane's offset), which keeps 64-bit
  // per-lane pointers out of the vector registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  TileCtx C;
  C.Fw = J.shared ? A.Fs : A.F;
  const int K = STAGE == 1 ? A.d : C.Fw;
  C.nk = K / KC;
  C.run = J.nb * WAVES + wave;
  // the ABI requires ffn widths % 128 and d % 256: every wave of a block has
  // a run of weight rows
  static_assert(WAVES * H_COLS_WAVE == H_COLS_BLOCK && WAVES * OUT_COLS_WAVE == OUT_COLS_BLOCK,
                "a block covers whole 64-row weight runs of every matrix");
  const size_t tb = tile_bytes(FMT);
  const uint8_t* blob = J.shared ? A.shared_blob
                                 : A.routed_blob + (size_t)J.expert * expert_bytes(FMT, A.d, A.F);
  C.sect = STAGE == 1 ? blob : blob + w1_bytes(FMT, A.d, C.Fw);
  C.wt = C.sect + (size_t)C.run * C.nk * tb;

  // Rows of this tile (thread m < ROWS has row m): source row of the
  // activations, folded router weight, fp16 row scale.  In stage 1 the first
  // PF weight chunks, which depend only on the expert, are issued right after
  // the row loads (so waiting for those does not wait for weights) instead of
  // after the row barrier; stage 2 rows need no loads.
  static_assert(ROWS <= WAVES * 64, "one row per thread");
  const int m = tid;
  int src = -1;
  float wf = 0.0f, xs = 1.0f;
  if (m < ROWS && m < J.cnt) {
    if (STAGE == 1) {
      if (J.shared) {
        src = J.start + m;
        wf = 1.0f;
      } else {
        const int f = A.perm[J.start + m];
        src = f / A.k;
        wf = A.topk_w[f];
      }
      if (F16) xs = A.xscale[src];
    } else {
      src = J.start + m;
    }
  }
  constexpr int PF = lead_of(FMT, PF_MAX);
  WTile<FMT> ring[PF];
  if constexpr (STAGE == 1) {
#pragma unroll
    for (int p = 0; p < PF; p++)
      ring[p].template load<NT>(BufSrc{buffer_rsrc(C.wt), (uint32_t)(p * tb)}, tid & 63);
  }
  if (m < ROWS) {
    sm.src[m] = src;
    sm.wrow[m] = wf;
    sm.xs[m] = xs;
  }
  __syncthreads();

  C.abase = STAGE == 1 ? (F16 ? (const uint8_t*)A.x16 : (const uint8_t*)A.hidden)
                       : (const uint8_t*)(J.shared ? A.h_shared : A.h_routed);
  // rows of 2-byte elements; every activation matrix is below 4 GiB (T*k <=
  // 2^30 rows of <= 16384 columns would not be: the ABI bounds T*k*ffn and
  // T*d to 2^31 elements)
  const uint32_t astride = STAGE == 1 ? (uint32_t)A.d : (uint32_t)C.Fw;
  // Rows past the tile's end load the tile's first row: their accumulator
  // rows are never stored, and every lane issues the same loads.
#pragma unroll
  for (int j = 0; j < PPT; j++) {
    const int q = (tid + WAVES * 64 * j) % PIECES;  // piece q: row q / 8, 16-byte chunk q % 8
    const int r = q >> 3;
    const int s = sm.src[r] >= 0 ? sm.src[r] : sm.src[0];
    C.aoff[j] = ((uint32_t)s * astride + (uint32_t)(q & 7) * 8) * 2;
  }
  tile_body<FMT, STAGE, MAXMF, PF_MAX, F16, NT>(A, J, sm, C, ring);
}

// A routed tile of a 96-row kernel with fewer rows runs a body with fewer row
// fragments (2, 4 or 5): the MFMAs of padding fragments are never issued, and
// the branch is taken once per tile, outside the MFMA stream.  Every body
// computes a row with the same MFMA chain and epilogue (row invariance).
// Measured at T=4096: grouped FFN -3.6% (about half the tiles hold <= 80
// rows; experts spilling past 96 rows leave small second tiles).
template <int RF, int STAGE, int MAXMF, int PF, bool F16, bool NT>
__device__ __forceinline__ void run_routed_tile(const FfnArgs& A, const TileJob& J,
                                                Smem<MAXMF, slots_of<RF, PF>()>& sm) {
  constexpr int SL = slots_of<RF, PF>();
  if constexpr (MAXMF == 6) {
    if (J.cnt <= 32)
      return run_tile<RF, STAGE, 2, PF, F16, NT>(A, J, *reinterpret_cast<Smem<2, SL>*>(&sm));
    if (J.cnt <= 64)
      return run_tile<RF, STAGE, 4, PF, F16, NT>(A, J, *reinterpret_cast<Smem<4, SL>*>(&sm));
    if (J.cnt <= 80)
      return run_tile<RF, STAGE, 5, PF, F16, NT>(A, J, *reinterpret_cast<Smem<5, SL>*>(&sm));
  }
  run_tile<RF, STAGE, MAXMF, PF, F16, NT>(A, J, sm);
}

// Grid: slot-major with the column block fastest *within an XCD*: block b runs
// on XCD b % 8; slot = (b / (8*NB)) * 8 + b % 8, nb = (b / 8) % NB.  So all
// column blocks of one row tile share an XCD (and its L2 copy of the gathered
// activation rows), and empty slots spread evenly over the XCDs.
// Slots to tiles: routed tiles in plan order, then the shared expert's tiles;
// slots past the plan's tiles are empty.  With SPREAD the shared tiles (which
// re-read one small weight set from cache and mostly compute) are instead
// spread evenly over the first L = shared + ceil(T*k / rows) slots -- a lower
// bound on the routed tiles in use -- between routed tiles, so they run beside
// tiles that stream their weights from HBM instead of forming the tail.  The
// MXFP4 kernels use it (routed tiles there do no dequantization: T=4096 and
// T=16 grouped FFN -4.6%); the int4 kernels do not (no gain, and the shared
// outputs then leave the cache before the combine reads them: +3 us there).
template <bool SPREAD = false>
__device__ __forceinline__ bool decode_job(const FfnArgs& A, int NB, int ncols_routed,
                                           int ncols_shared, int rows_per_tile, TileJob& J) {
  const int b = blockIdx.x;
  const int slot = (b / (8 * NB)) * 8 + (b & 7);
  J.nb = (b >> 3) % NB;
  const int ns = A.shared_slots, S = A.routed_slots + ns;
  if (slot >= S) return false;
  const int L = SPREAD ? min(S, ns + (A.T * A.k + rows_per_tile - 1) / rows_per_tile) : S;
  int routed = SPREAD ? slot - ns : slot;
  if (!SPREAD && slot >= A.routed_slots) {
    J.shared = true;
    J.expert = -1;
    J.start = (slot - A.routed_slots) * rows_per_tile;
    J.cnt = min(rows_per_tile, A.T - J.start);
    return J.nb < ncols_shared;
  }
  if (SPREAD && slot < L) {
    const int before = (int)((int64_t)slot * ns / L);  // shared tiles in slots [0, slot)
    if ((int)((int64_t)(slot + 1) * ns / L) > before) {
      J.shared = true;
      J.expert = -1;
      J.start = before * rows_per_tile;
      J.cnt = min(rows_per_tile, A.T - J.start);
      return J.nb < ncols_shared;
    }
    routed = slot - before;
  }
  const int4 t = A.tiles[routed];  // one scalar load: (expert, first row, rows)
  if (t.z == 0) return false;
  J.shared = false;
  J.expert = t.x;
  J.start = t.y;
  J.cnt = min(rows_per_tile, t.z);
  return J.nb < ncols_routed;
}

// column blocks of a matrix with `runs` 64-row weight runs
__host__ __device__ __forceinline__ int col_blocks(int runs) { return (runs + WAVES - 1) / WAVES; }

template <int RF, int SF, int STAGE, int MAXMF, int PF, bool NT_ROUTED>
__global__ __launch_bounds__(WAVES * 64, 8 / WAVES) void ffn_kernel(FfnArgs A) {
  __shared__ __attribute__((aligned(16))) Smem<MAXMF, slots_of<RF, PF>()> sm;
  const int nr = STAGE == 1 ? col_blocks(A.F / H_COLS_WAVE) : col_blocks(A.d / OUT_COLS_WAVE);
  const int ns = STAGE == 1 ? (A.n_shared ? col_blocks(A.Fs / H_COLS_WAVE) : 0) : nr;
  TileJob J;
  if (!decode_job(A, max(nr, ns), nr, ns, MAXMF * 16, J)) return;
  // int4 routed layers run gate/up on fp16 MFMA (the fp16 activation copy
  // exists); int8 shared tiles of such a layer follow; bf16 weights stay bf16
  constexpr bool X16 = x16_path(RF, MAXMF);
  // NT_ROUTED: routed weights streamed past the caches (non-temporal).  The
  // shared expert's weights are re-read by every row tile: those stay
  // cacheable.
  constexpr bool NT_SHARED = false;
  static_assert(slots_of<SF, PF>() <= slots_of<RF, PF>(), "shared tiles fit the routed LDS");
  if (J.shared)
    run_tile<SF, STAGE, MAXMF, PF, STAGE == 1 && X16 && SF == MOE_I8_ROW, NT_SHARED>(
        A, J, *reinterpret_cast<Smem<MAXMF, slots_of<SF, PF>()>*>(&sm));
  else
    run_routed_tile<RF, STAGE, MAXMF, PF, STAGE == 1 && X16, NT_ROUTED>(A, J, sm);
}

// Row tiles come from the route plan, cut at tile_rows(T) rows: a call with
// at most 16 or 32 tokens runs a kernel built for 1 or 2 row fragments with a
// deeper weight prefetch (shared-expert tiles then hold 16 or 32 tokens), a
// larger call 96-row tiles.
template <int RF, int SF, int MAXMF, int PF, bool NT_ROUTED>
static hipError_t launch_stages(const FfnArgs& a0, hipStream_t s) {
  FfnArgs a = a0;
  a.shared_slots = a.n_shared ? (a.T + MAXMF * 16 - 1) / (MAXMF * 16) : 0;
  const int slots = (a.routed_slots + a.shared_slots + 7) / 8 * 8;
  const int nb1 = col_blocks(max(a.F, a.n_shared ? a.Fs : 0) / H_COLS_WAVE);
  const int nb2 = col_blocks(a.d / OUT_COLS_WAVE);
  // the fp16 copy of x of int4 / b-bit layers comes from moe_permute's plan
  ffn_kernel<RF, SF, 1, MAXMF, PF, NT_ROUTED><<<slots * nb1, WAVES * 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_kernel<RF, SF, 2, MAXMF, PF, NT_ROUTED><<<slots * nb2, WAVES * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Routed weights are streamed past the caches when the call averages at most
// one row tile per expert (every small-T call; T=4096 at k=10 of 512): each
// expert's weights are then read about once, and keeping them out of L2 and
// the MALL leaves room for the gathered activation rows and for the fp32
// outputs the combine reads next (T=4096: combine 82 -> 73 us; bf16 weights
// at T=512: grouped FFN -7%).  With more rows per expert its tiles re-read
// its weights, which then stay cacheable (T=16384 streamed: +2%).
template <int RF, int SF>
static hipError_t launch_pair(const FfnArgs& a, hipStream_t s) {
  static_assert(tile_rows(16) == 16 && tile_rows(32) == 32 && tile_rows(33) == BM,
                "kernel choice follows the route plan's tile rows");
  if (a.T <= 16) return launch_stages<RF, SF, 1, LEAD_I4, true>(a, s);
  if (a.T <= 32) return launch_stages<RF, SF, 2, LEAD_I4, true>(a, s);
  if ((int64_t)a.T * a.k <= (int64_t)a.E * BM)
    return launch_stages<RF, SF, BM / 16, LEAD_I4, true>(a, s);
  return launch_stages<RF, SF, BM / 16, LEAD_I4, false>(a, s);
}

}  // namespace moe
