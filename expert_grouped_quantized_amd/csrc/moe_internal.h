// moe_internal.h -- layout constants and launch entry points shared by the
// host side (abi.cpp, the packer) and the HIP kernels.  Not installed; the
// public interface is include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---- tiling of the expert-grouped GEMMs (MFMA 16x16x32) ----------------
// A block is 4 wave64s.  It owns up to BM rows of one expert's group; each
// wave owns one run of 64 weight rows:
//   stage 1 (gate/up): 32 h columns = 32 gate rows + 32 up rows of W1, so a
//                      block makes 128 h columns;
//   stage 2 (down):    64 output columns, a block 256.
// K advances in chunks of KC; one chunk of one wave's 64 weight rows is a
// "wave tile", stored contiguously in the blob; the blob orders wave tiles by
// run index, then K chunk, independent of the block shape.
constexpr int BM = 96;             // rows of an expert group per row tile (6 x 16)
constexpr int KC = 64;             // K per chunk (2 MFMA K-steps of 32)
constexpr int WAVES = 4;           // waves per GEMM block
constexpr int H_COLS_WAVE = 32;    // stage-1 h columns per wave run
constexpr int OUT_COLS_WAVE = 64;  // stage-2 output columns per wave run
constexpr int H_COLS_BLOCK = 128;    // the layer's ffn widths are multiples of this
constexpr int OUT_COLS_BLOCK = 256;  // the layer's hidden width is a multiple of this
// K chunks each wave keeps in flight: int4 weight tiles, and the wider bf16
// and int8 ones.  A matrix's K must be a multiple of KC times its lead.
constexpr int LEAD_I4 = 4;
constexpr int LEAD_WIDE = 2;

// wave-tile bytes (64 weight rows x 64 K) per stored format
constexpr int TILE_BYTES_BF16 = 64 * 64 * 2;        // 8192
constexpr int TILE_BYTES_I4 = 64 * 64 / 2 + 64 * 2 * 2;  // 2048 codes + 256 scales
constexpr int TILE_BYTES_I8 = 64 * 64;              // 4096 (row scales kept apart)
// MXFP4 (scaled FP4 MFMA 16x16x128): a wave tile is 64 weight rows x 128 K,
// 4096 bytes of e2m1 codes + 256 E8M0 scale bytes; its K loop keeps
// LEAD_MX chunks in flight
constexpr int KC_MX = 128;
constexpr int TILE_BYTES_MX4 = 64 * 128 / 2 + 64 * 4;  // 4352
constexpr int LEAD_MX = 2;

// Rows of a routed row tile in a call of T tokens.  moe_permute cuts every
// expert's group into tiles of this many rows and moe_grouped_ffn launches the
// kernels built for that tile: one or two 16-row fragments for calls of at most
// 16 or 32 tokens, BM rows above.  A group can outgrow T (a caller's ids may
// name one expert twice for a token), so the cut must not assume it cannot.
__host__ __device__ constexpr int tile_rows(int64_t T) { return T <= 16 ? 16 : T <= 32 ? 32 : BM; }

// ---- route plan ----------------------------------------------------------
constexpr int PLAN_CHUNK = 1024;   // assignments per block of the plan kernels
constexpr int PLAN_THREADS = 1024; // 16 waves
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_TOPK = 32;

// Bits per code of the group-32 integer formats (4 for MOE_I4_G32), else 0.
__host__ __device__ constexpr int ig32_bits(int fmt) {
  return fmt == MOE_I4_G32 ? 4 : fmt == MOE_I2_G32 ? 2 : fmt == MOE_I3_G32 ? 3
       : fmt == MOE_I5_G32 ? 5 : fmt == MOE_I6_G32 ? 6 : fmt == MOE_I7_G32 ? 7
       : fmt == MOE_I8_G32 ? 8 : 0;
}
// b-bit group-32 wave tile: 64 lanes x 8b bytes of codes, then the 256 bytes
// of fp16 group scales (b = 4 gives the int4 tile's 2304 bytes)
__host__ __device__ constexpr int tile_bytes_ig32(int b) { return 512 * b + 256; }

__host__ __device__ inline size_t tile_bytes(int fmt) {
  return fmt == MOE_BF16 ? TILE_BYTES_BF16
       : fmt == MOE_I4_G32 ? TILE_BYTES_I4
       : fmt == MOE_I8_ROW ? TILE_BYTES_I8
       : fmt == MOE_MXFP4 ? TILE_BYTES_MX4
       : tile_bytes_ig32(ig32_bits(fmt));
}
// K of one wave tile
__host__ __device__ constexpr int kc_of(int fmt) { return fmt == MOE_MXFP4 ? KC_MX : KC; }
// K chunks each wave keeps in flight for a weight format: 4- and 2-bit codes
// take LEAD_I4, the other tiles LEAD_WIDE (their registers; a lead of 4 for
// 3-bit codes in the 16- and 32-row tiles measured slower at T=16)
__host__ __device__ constexpr int lead_of(int fmt, int lead_i4) {
  return fmt == MOE_MXFP4 ? LEAD_MX
       : (ig32_bits(fmt) == 4 || ig32_bits(fmt) == 2) ? lead_i4 : LEAD_WIDE;
}

// Bytes of the W1 (gate/up, [2F, d]) and W2 (down, [d, F]) sections of one
// expert in the device blob.
__host__ __device__ inline size_t w1_bytes(int fmt, size_t d, size_t F) {
  if (fmt == MOE_F32) return 2 * F * d * 4;
  size_t tiles = (2 * F / 64) * (d / kc_of(fmt)) * tile_bytes(fmt);  // 64-row wave tiles
  return tiles + (fmt == MOE_I8_ROW ? 2 * F * 2 : 0);
}
__host__ __device__ inline size_t w2_bytes(int fmt, size_t d, size_t F) {
  if (fmt == MOE_F32) return d * F * 4;
  size_t tiles = (d / 64) * (F / kc_of(fmt)) * tile_bytes(fmt);
  return tiles + (fmt == MOE_I8_ROW ? d * 2 : 0);
}
__host__ __device__ inline size_t expert_bytes(int fmt, size_t d, size_t F) {
  return w1_bytes(fmt, d, F) + w2_bytes(fmt, d, F);
}

// Workspace layout, shared by moe_workspace_bytes, moe_permute and
// moe_grouped_ffn.  Every region starts on a 256-byte boundary.
struct WsLayout {
  size_t ticket;       // int32 [4] at offset 0 for every T: the block counters
                       //                       of moe_route_plan's one-launch form, zero
                       //                       between calls (no other call writes them)
  int n_chunks;        // plan blocks
  int routed_slots;    // upper bound on routed row tiles
  size_t counts;       // int32 [n_chunks][E]   per-chunk expert histogram
  size_t tiles;        // int4  [routed_slots]  (expert, first row, rows, 0) per
                       //                       tile; rows 0 past the plan's tiles
  size_t h_routed;     // act-typed [T*k, F]    intermediate h, permuted rows
                       //   (MXFP4 layers: e2m1 codes [T*k, F/2], chunk-major)
  size_t h_scale;      // MXFP4 layers: E8M0 [T*k, F/32], the scales of h
  size_t h_shared;     // act-typed [T, Fs]     intermediate h of the shared expert
  size_t x16;          // fp16 [T, d]           activations scaled by 2^-xexp[t] (int4 / b-bit
                       //                       layers; written by moe_permute)
                       //   (MXFP4 layers: e2m1 codes of x in plan order [T*k, d/2])
  size_t xexp;         // float [T]             2^xexp[t], the scale to undo
                       //   (MXFP4 layers: E8M0 [T*k, d/32], the scales of x)
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WsLayout ws_layout(const moe_desc& D, int64_t T, int64_t k) {
  WsLayout L{};
  int64_t n = T * k;
  L.n_chunks = (int)((n + PLAN_CHUNK - 1) / PLAN_CHUNK);
  const int64_t R = tile_rows(T);
  int64_t bound = (n + R - 1) / R + (n < D.n_experts ? n : D.n_experts);
  L.routed_slots = (int)(bound < n ? bound : n);
  size_t elem = D.act == MOE_F32 ? 4 : 2;
  size_t off = 0;
  L.ticket = off;   off = align256(off + 16);
  L.counts = off;   off = align256(off + (size_t)L.n_chunks * D.n_experts * 4);
  L.tiles = off;    off = align256(off + (size_t)L.routed_slots * 16);
  const bool mx = D.act == MOE_BF16 && D.expert_w == MOE_MXFP4;
  L.h_routed = off; off = align256(off + (size_t)n * D.ffn * (mx ? 1 : 2 * elem) / 2);
  L.h_scale = off;  off = align256(off + (mx ? (size_t)n * (D.ffn / 32) : 0));
  L.h_shared = off; off = align256(off + (D.n_shared ? (size_t)T * D.shared_ffn * elem : 0));
  const bool x16 = D.act == MOE_BF16 && ig32_bits(D.expert_w) != 0;
  L.x16 = off;      off = align256(off + (x16 ? (size_t)T * D.d * 2 : mx ? (size_t)n * D.d / 2 : 0));
  L.xexp = off;     off = align256(off + (x16 ? (size_t)T * 4 : mx ? (size_t)n * (D.d / 32) : 0));
  L.total = off;
  return L;
}

// ---- launches (each returns the HIP error of its launch) ------------------
hipError_t launch_router_bf16(int T, int d, int E, const void* x, const void* wr, const float* bias,
                              float* logits, hipStream_t s);
hipError_t launch_router_f32(int T, int d, int E, const float* x, const float* wr,
                             const float* bias, float* logits, hipStream_t s);
hipError_t launch_topk(int T, int E, int k, const float* logits, int32_t* ids, float* w,
                       hipStream_t s);
// Route plan of T*k ids, tiles of `rows` rows.  x_for_f16 (int4 / b-bit
// layers, else NULL): also write the fp16 copy of x (rows of d, each scaled
// by a power of two) and its per-token scales into the workspace.
hipError_t launch_plan(int T, int k, int E, int rows, const int32_t* ids, int32_t* offsets,
                       int32_t* perm, int32_t* inv_perm, void* ws, const WsLayout& L, int d,
                       const uint16_t* x_for_f16, hipStream_t s);
// Router, top-k, plan and (with_x16) the fp16 copy of x in one launch, for
// bf16 calls of at most 32 tokens (route_plan.hip); the workspace's counters
// must be zero, and are zero again when the launch ends.
hipError_t launch_route_plan_small(int T, int d, int E, int k, const void* x, const void* wr,
                                   const float* bias, float* logits, int32_t* ids, float* w,
                                   int32_t* offsets, int32_t* perm, int32_t* inv_perm, int rows,
                                   void* ws, const WsLayout& L, bool with_x16, hipStream_t s);


struct FfnArgs {
  int T, k, d, E, F, Fs, n_shared;
  int routed_fmt, shared_fmt;
  int routed_slots, shared_slots;
  const void* hidden;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* perm;
  const int4* tiles;
  const uint8_t* routed_blob;
  const uint8_t* shared_blob;
  void* h_routed;
  void* h_shared;
  uint16_t* x16;    // fp16 activations of the int4 path (workspace)
  float* xscale;    // per-token power of two undone in the gate/up epilogue
  // MXFP4 layers (workspace): e2m1 codes and E8M0 scales of x and of h
  uint8_t* xq;
  uint8_t* xsc;
  uint8_t* hq;
  uint8_t* hsc;
  float* out_assign;
  float* shared_out;
};
hipError_t launch_ffn_bf16(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s);
// routed weights in the 2, 3, 5, 6, 7 or 8-bit group-32 formats
hipError_t launch_ffn_lowbit(const FfnArgs& a, hipStream_t s);
// MXFP4 W4A4 routed experts
hipError_t launch_ffn_mx(const FfnArgs& a, hipStream_t s);
hipError_t launch_combine(int T, int k, int d, int act, const float* out_assign,
                          const int32_t* inv_perm, const float* shared_out, void* y,
                          hipStream_t s);
// the route plan's row tiles rebuilt from its offsets alone (and, x given,
// the fp16 copy of x and its per-token scales)
hipError_t launch_tiles_from_offsets(int E, int rows, int slots, const int32_t* offsets,
                                     int4* tiles, int T, int d, const uint16_t* x,
                                     uint16_t* x16, float* xscale, hipStream_t s);

// moe_grouped_ffn's checks and launches.  With scratch == nullptr the
// intermediates go to the caller's workspace `ws` of ws_bytes, where
// moe_permute left the row-tile plan.  Otherwise `ws` is ignored: once every
// argument has passed its checks and T > 0, scratch() gives the address of a
// library-held region of ws_bytes (moe_grouped_ffn_noalloc), and the row-tile
// plan is first rebuilt there from `offsets`.
typedef hipError_t (*ScratchFn)(void** address);
moe_status grouped_ffn_call(const moe_desc* D, int32_t T, int32_t k, const void* hidden,
                            const float* topk_w, const int32_t* offsets, const int32_t* perm,
                            const void* routed_blob, const void* shared_blob, float* out_assign,
                            float* shared_out, void* ws, size_t ws_bytes, ScratchFn scratch,
                            void* stream);

}  // namespace moe
