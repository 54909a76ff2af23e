// permute.hip -- the route plan: every assignment ordered by expert, the same
// order on every run
// ("Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated prefill lane",
// step 1; TandemLLM docs 17.4: a chunk sorts its (row, expert) pairs by expert).
//
// offsets = exclusive prefix sum of the expert histogram; perm = a stable
// counting sort of the flat assignment index f = t*k + s by expert (ascending f
// inside each expert); inv_perm its inverse.  The input is cut into chunks of
// PLAN_CHUNK (= the block size, so one rank pass each) assignments, one
// 1024-thread block each:
//   plan_count   : per-chunk histogram in LDS -> counts[chunk][E]
//   plan_scatter : totals and per-chunk bases from counts (fixed order), block
//                  scan -> offsets; stable in-chunk ranks from wave ballots
//                  (lanes holding the same expert id) plus per-wave counts in
//                  LDS; perm/inv_perm scattered; chunk 0 also writes offsets
//                  and the row-tile plan for the grouped GEMMs.
// For int4 / b-bit layers the plan_scatter launch also carries blocks that
// write the fp16 copy of x the grouped gate/up products run on (see
// x16_blocks).
// Only the histogram uses atomics, and counts do not depend on their order;
// every position is a function of the input alone.
#include "plan_kernels.h"

namespace moe {

// Blocks past the plan's own that write the fp16 copy of an int4 (or b-bit)
// layer's activations and its per-token scales (x given): one wave per token.
// They share the plan_scatter launch (they need nothing from the plan), so
// the copy costs no launch of its own and runs beside the plan's few blocks
// (T=4096: 256 blocks beside 40; permute 22.0 -> 20.1 us against carrying
// them in plan_count, whose histogram blocks finish first).
constexpr int X16_TOKENS_PER_BLOCK = PLAN_THREADS / 64;
inline int x16_blocks(int T, const uint16_t* x) {
  return x ? (T + X16_TOKENS_PER_BLOCK - 1) / X16_TOKENS_PER_BLOCK : 0;
}

// One chunk's histogram per block.
__global__ __launch_bounds__(PLAN_THREADS) void plan_count_kernel(
    int n, int E, const int32_t* __restrict__ ids, int32_t* __restrict__ counts) {
  __shared__ int hist[MAX_EXPERTS];
  const int tid = threadIdx.x, base = blockIdx.x * PLAN_CHUNK;
  const int len = min(PLAN_CHUNK, n - base);
  for (int e = tid; e < E; e += PLAN_THREADS) hist[e] = 0;
  __syncthreads();
  for (int i = tid; i < len; i += PLAN_THREADS) atomicAdd(&hist[ids[base + i]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += PLAN_THREADS) counts[(size_t)blockIdx.x * E + e] = hist[e];
}


// The row tiles alone, from a finished plan's offsets (block 0), and the
// fp16 copy of x (blocks past it, when x is given).
__global__ __launch_bounds__(PLAN_THREADS) void tiles_from_offsets_kernel(
    int E, int rows, int slots, const int32_t* __restrict__ offsets, int4* __restrict__ tiles,
    int T, int d, const uint16_t* __restrict__ x, uint16_t* __restrict__ x16,
    float* __restrict__ xscale) {
  __shared__ int wsum[PLAN_WAVES];
  __shared__ int total_all;
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    rows_to_f16(T, d, x, x16, xscale, (blockIdx.x - 1) * X16_TOKENS_PER_BLOCK + (tid >> 6),
                (gridDim.x - 1) * X16_TOKENS_PER_BLOCK);
    return;
  }
  const int off = tid < E ? offsets[tid] : 0;
  const int total = tid < E ? offsets[tid + 1] - off : 0;
  write_row_tiles(E, rows, slots, total, off, wsum, &total_all, tiles);
}

hipError_t launch_tiles_from_offsets(int E, int rows, int slots, const int32_t* offsets,
                                     int4* tiles, int T, int d, const uint16_t* x,
                                     uint16_t* x16, float* xscale, hipStream_t s) {
  tiles_from_offsets_kernel<<<1 + x16_blocks(T, x), PLAN_THREADS, 0, s>>>(
      E, rows, slots, offsets, tiles, T, d, x, x16, xscale);
  return hipGetLastError();
}

// One chunk per block; blocks past the chunks write the fp16 copy of x (x
// given; see x16_blocks).
template <bool SINGLE>
__global__ __launch_bounds__(PLAN_THREADS) void plan_scatter_kernel(
    int n, int E, int n_chunks, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int rows, int slots, int4* __restrict__ tiles, int T, int d,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ x16, float* __restrict__ xscale) {
  __shared__ PlanSmem sm;
  const int nplan = SINGLE ? 1 : n_chunks;
  if ((int)blockIdx.x >= nplan) {
    rows_to_f16(T, d, x, x16, xscale,
                ((int)blockIdx.x - nplan) * X16_TOKENS_PER_BLOCK + (threadIdx.x >> 6),
                ((int)gridDim.x - nplan) * X16_TOKENS_PER_BLOCK);
    return;
  }
  plan_scatter_block<SINGLE>(n, E, n_chunks, blockIdx.x, ids, counts, offsets, perm, inv_perm,
                             rows, slots, tiles, sm);
}

hipError_t launch_plan(int T, int k, int E, int rows, const int32_t* ids, int32_t* offsets,
                       int32_t* perm, int32_t* inv_perm, void* ws, const WsLayout& L, int d,
                       const uint16_t* x_for_f16, hipStream_t s) {
  const int n = T * k;
  uint8_t* w = (uint8_t*)ws;
  int32_t* counts = (int32_t*)(w + L.counts);
  int4* tiles = (int4*)(w + L.tiles);
  float* xscale = (float*)(w + L.xexp);
  uint16_t* x16 = (uint16_t*)(w + L.x16);
  if (L.n_chunks == 1) {
    plan_scatter_kernel<true><<<1 + x16_blocks(T, x_for_f16), PLAN_THREADS, 0, s>>>(
        n, E, 1, ids, counts, offsets, perm, inv_perm, rows, L.routed_slots, tiles, T, d,
        x_for_f16, x16, xscale);
  } else {
    plan_count_kernel<<<L.n_chunks, PLAN_THREADS, 0, s>>>(n, E, ids, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    plan_scatter_kernel<false><<<L.n_chunks + x16_blocks(T, x_for_f16), PLAN_THREADS, 0, s>>>(
        n, E, L.n_chunks, ids, counts, offsets, perm, inv_perm, rows, L.routed_slots, tiles, T, d,
        x_for_f16, x16, xscale);
  }
  return hipGetLastError();
}

}  // namespace moe
