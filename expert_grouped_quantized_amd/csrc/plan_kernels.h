// plan_kernels.h -- the route plan's block-level pieces (fixed-order scan,
// row tiles, the stable scatter of one chunk) as device functions.
// See permute.hip for what the plan is and where the pages describe it.
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int PLAN_WAVES = PLAN_THREADS / 64;  // 16

// Exclusive scan of one int per thread over a 1024-thread block (fixed order).
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < PLAN_WAVES; w++) {
      int t = wsum[w];
      wsum[w] = acc;
      acc += t;
    }
    *total = acc;
  }
  __syncthreads();
  int r = wsum[wave] + incl - v;
  __syncthreads();
  return r;
}

// Row tiles of the grouped GEMMs (thread e < E holds expert e's row count
// `total` and first row `off`): expert e owns ceil(total / rows) tiles, each
// stored resolved as (expert, first row, rows) so a GEMM block finds its rows
// with one load; the slots past the plan's tiles, up to `slots`, get 0 rows.
// Every thread of the block must call it.
__device__ __forceinline__ void write_row_tiles(int E, int rows, int slots, int total, int off, int* wsum,
                                int* total_all, int4* __restrict__ tiles) {
  const int tid = threadIdx.x;
  const int nt = tid < E ? (total + rows - 1) / rows : 0;
  const int tstart = block_exclusive_scan(nt, wsum, total_all);
  for (int j = 0; j < nt; j++)
    tiles[tstart + j] = make_int4(tid, off + j * rows, min(rows, total - j * rows), 0);
  for (int j = *total_all + tid; j < slots; j += PLAN_THREADS) tiles[j] = make_int4(0, 0, 0, 0);
}

// LDS of one plan block.
struct PlanSmem {
  int run[MAX_EXPERTS];
  int hist[MAX_EXPERTS];
  __attribute__((aligned(16))) uint8_t wcnt[PLAN_WAVES][MAX_EXPERTS];
  int wsum[PLAN_WAVES];
  int total_all;
};

// Chunk `chunk` of the route plan, by one block of PLAN_THREADS threads.
// SINGLE: the whole plan is one chunk (n <= PLAN_CHUNK) and its histogram is
// taken here instead of read from `counts`.
template <bool SINGLE>
__device__ void plan_scatter_block(int n, int E, int n_chunks, int chunk,
                                   const int32_t* __restrict__ ids,
                                   const int32_t* __restrict__ counts,
                                   int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                   int32_t* __restrict__ inv_perm, int rows, int slots,
                                   int4* __restrict__ tiles, PlanSmem& sm) {
  int* run = sm.run;
  int* hist = sm.hist;
  auto& wcnt = sm.wcnt;
  int* wsum = sm.wsum;
  int& total_all = sm.total_all;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = chunk * PLAN_CHUNK;
  const int len = min(PLAN_CHUNK, n - base);

  // 1) this expert's total and the part of it in earlier chunks
  int before = 0, total = 0;
  if (SINGLE) {
    for (int e = tid; e < E; e += PLAN_THREADS) hist[e] = 0;
    __syncthreads();
    for (int i = tid; i < len; i += PLAN_THREADS) atomicAdd(&hist[ids[base + i]], 1);
    __syncthreads();
    if (tid < E) total = hist[tid];
  } else {
    // PLAN_THREADS / E threads per expert each sum every r-th chunk's count;
    // the parts are then added through LDS (integer sums: order-free)
    const int r = PLAN_THREADS / E, e = tid % E, part = tid / E;
    if (part < r) {
      // eight chunks' counts a batch, loaded with no condition (indices past
      // the last chunk re-read it and are not added) so they are in flight
      // together
      for (int c0 = part; c0 < n_chunks; c0 += 8 * r) {
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = counts[(size_t)min(c0 + j * r, n_chunks - 1) * E + e];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const int c = c0 + j * r;
          if (c < n_chunks) {
            if (c < chunk) before += v[j];
            total += v[j];
          }
        }
      }
    }
    hist[tid] = total;
    run[tid] = before;
    __syncthreads();
    if (tid < E) {
      for (int q = 1; q < r; q++) {
        total += hist[tid + q * E];
        before += run[tid + q * E];
      }
    }
    __syncthreads();
  }
  // 2) offsets
  const int off = block_exclusive_scan(tid < E ? total : 0, wsum, &total_all);
  if (tid < E) run[tid] = off + before;
  if (chunk == 0) {
    if (tid < E) offsets[tid] = off;
    if (tid == 0) offsets[E] = n;
    // 3) row tiles of the grouped GEMMs
    write_row_tiles(E, rows, slots, total, off, wsum, &total_all, tiles);
  }
  __syncthreads();

  // 4) stable scatter, 1024 assignments at a time
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const uint64_t gt_mask = lane == 63 ? 0ull : ~((2ull << lane) - 1ull);
  int nbits = 0;
  while ((1 << nbits) < E) nbits++;
  for (int sub = 0; sub < len; sub += PLAN_THREADS) {
    const int i = sub + tid;
    const bool valid = i < len;
    const int id = valid ? ids[base + i] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; b++) {
      uint64_t bb = __ballot((id >> b) & 1);
      same &= ((id >> b) & 1) ? bb : ~bb;
    }
    // clear the per-wave counts (16 KB: one 16-byte store per thread)
    ((u32x4_t*)&wcnt[0][0])[tid] = u32x4_t{0, 0, 0, 0};
    __syncthreads();
    const int rank_w = __popcll(same & lt_mask);
    if (valid && rank_w == 0) wcnt[wave][id] = (uint8_t)__popcll(same);
    __syncthreads();
    int pos = 0;
    bool last = false;
    if (valid) {
      int pre = 0, post = 0;
      for (int w2 = 0; w2 < PLAN_WAVES; w2++) {
        int c = wcnt[w2][id];
        if (w2 < wave) pre += c;
        if (w2 > wave) post += c;
      }
      pos = run[id] + pre + rank_w;
      perm[pos] = base + i;
      inv_perm[base + i] = pos;
      last = ((same & gt_mask) == 0ull) && post == 0;
    }
    __syncthreads();
    if (valid && last) run[id] = pos + 1;
    __syncthreads();
  }
}

}  // namespace moe
