// route_plan.hip -- the front end of a small call (T <= 32 tokens, bf16
// activations) in one launch: router logits, the stable top-k and softmax,
// the route plan with its row tiles, and the fp16 copy of x.
//
// What each part computes, and where the pages say it, is as in route.hip
// (router, top-k) and permute.hip (plan); this file only joins them.  The
// pages price a joint pass over up to 32 rows against a 16-row one
// (TandemLLM Roadmap v0.11.2, "Parallel requests"; TandemLLM docs 17.5
// "Speculation"): a call that small is bound by launches and latency, so the
// layer's front end is one kernel.
//
// Grid: the tokens fall into groups of 16 (one MFMA row fragment; two groups
// at most), and each group has one 1024-thread block per 16 experts.  In each
// block waves 0-7 make the logits of its 16 experts for the group's tokens
// (router_small_block: the router kernel's summation, so the logits are
// bit-identical), while waves 8-15 write fp16 rows of x (int4 / b-bit
// layers).  Each block then takes a ticket from its group's counter in the
// workspace; the group's last block -- every logit of its tokens is then
// written -- runs their top-k, one token a wave.  The route plan of all T * k
// assignments (plan_scatter_block, one chunk, in LDS) follows in that block
// when there is one group, else in the group whose top-k finishes last (a
// second ticket).  The last block sets every counter back to zero for the
// next call.  The results equal those of the separate route and permute
// launches bit for bit.  (Groups of 16 keep the serial part short: one block
// ranking all 32 tokens of a call, two a wave, took 8 us against 4.7 for 16.)
//
// Ordering: a block's stores complete before its barrier; one thread then
// makes them visible at agent scope (release fence) before taking a ticket,
// and the block that draws a counter's last ticket acquires at agent scope
// before its barrier and its loads.
#include "plan_kernels.h"
#include "route_kernels.h"

namespace moe {

constexpr int RP_THREADS = 1024;  // 16 waves: 8 router waves, 8 fp16-copy waves
static_assert(RP_THREADS == PLAN_THREADS, "the last block runs the plan's block code");
static_assert(RS_WAVES == 8, "waves 0-7 of a block are the router's eight K slices");
constexpr int RP_MAX_T = 32;  // the largest call it serves

// Counters at the start of the workspace (zero between calls): one per
// 16-token group, then one for the groups' top-k blocks.
constexpr int RP_GROUP = 16;  // tokens of one router block's group (one MFMA fragment)
constexpr int RP_CTR_DONE = RP_MAX_T / RP_GROUP;
static_assert(RP_CTR_DONE < 4, "the counters fit the workspace's first 16 bytes");

// Takes a ticket from *ctr (thread 0; the block's stores are complete at the
// barrier before) and says whether it was the last of n; the last block
// acquires what the others released.
__device__ __forceinline__ bool last_to_arrive(int* ctr, int n, int* flag) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int t = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = t == n - 1;
    if (*flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *flag;
}

template <int PL>
__global__ __launch_bounds__(RP_THREADS) void route_plan_small_kernel(
    int T, int d, int E, int k, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int rows, int slots, int4* __restrict__ tiles,
    uint16_t* __restrict__ x16, float* __restrict__ xscale, int* __restrict__ ctr) {
  // the router's partial tiles are dead before the plan's LDS is first used
  __shared__ union {
    f32x4_t part[RS_WAVES][1][64];
    PlanSmem plan;
  } sm;
  __shared__ int32_t ids_lds[RP_GROUP * MAX_TOPK];
  __shared__ int flag;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int groups = (T + RP_GROUP - 1) / RP_GROUP;
  const int neb = (int)gridDim.x / groups;  // router blocks of one token group
  const int g = (int)blockIdx.x / neb, eb = (int)blockIdx.x % neb;
  const int t0 = g * RP_GROUP;

  // 1) logits of 16 experts for the group's tokens (waves 0-7) beside fp16
  //    rows of x (waves 8-15, at most one token each); the copy waves meet
  //    the router waves' one internal barrier with one of their own
  if (wave < RS_WAVES) {
    router_small_block<1>(T, d, E, x, wr, bias, logits, eb * RS_EXPERTS, t0, wave, sm.part,
                          [] { __syncthreads(); });
  } else {
    if (x16)
      rows_to_f16(T, d, x, x16, xscale,
                  blockIdx.x * (RP_THREADS / 64 - RS_WAVES) + wave - RS_WAVES,
                  gridDim.x * (RP_THREADS / 64 - RS_WAVES));
    __syncthreads();
  }
  __syncthreads();  // each wave has waited for its logit stores

  // 2) the last router block of the group: top-k and softmax of its tokens,
  //    one a wave
  if (!last_to_arrive(ctr + g, neb, &flag)) return;
  const int t = t0 + wave;
  if (wave < RP_GROUP && t < T) {
    float lv[PL];
    topk_load<PL>(t, E, logits, lv);
    topk_select<PL>(t, E, k, lv, ids, w, ids_lds, wave);
  }
  __syncthreads();

  // 3) the route plan of the T * k ids, by the group's block when there is
  //    one group, else by the last group to finish its top-k (ids read back
  //    from memory)
  const int32_t* plan_ids = ids_lds;
  if (groups > 1) {
    if (!last_to_arrive(ctr + RP_CTR_DONE, groups, &flag)) return;
    plan_ids = ids;
  }
  plan_scatter_block<true>(T * k, E, 1, 0, plan_ids, nullptr, offsets, perm, inv_perm, rows, slots,
                           tiles, sm.plan);
  // every counter is back to zero when the launch ends: each group's last
  // ticket and the groups' last ticket were drawn before this point
  if (tid <= RP_CTR_DONE) ctr[tid] = 0;
}

hipError_t launch_route_plan_small(int T, int d, int E, int k, const void* x, const void* wr,
                                   const float* bias, float* logits, int32_t* ids, float* w,
                                   int32_t* offsets, int32_t* perm, int32_t* inv_perm, int rows,
                                   void* ws, const WsLayout& L, bool with_x16, hipStream_t s) {
  uint8_t* b = (uint8_t*)ws;
  int4* tiles = (int4*)(b + L.tiles);
  uint16_t* x16 = with_x16 ? (uint16_t*)(b + L.x16) : nullptr;
  float* xscale = with_x16 ? (float*)(b + L.xexp) : nullptr;
  int* ctr = (int*)(b + L.ticket);
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)wr;
  const int groups = (T + RP_GROUP - 1) / RP_GROUP;
  const int blocks = groups * ((E + RS_EXPERTS - 1) / RS_EXPERTS);
  if (E <= 8 * 64)
    route_plan_small_kernel<8><<<blocks, RP_THREADS, 0, s>>>(
        T, d, E, k, xp, wp, bias, logits, ids, w, offsets, perm, inv_perm, rows, L.routed_slots,
        tiles, x16, xscale, ctr);
  else
    route_plan_small_kernel<16><<<blocks, RP_THREADS, 0, s>>>(
        T, d, E, k, xp, wp, bias, logits, ids, w, offsets, perm, inv_perm, rows, L.routed_slots,
        tiles, x16, xscale, ctr);
  return hipGetLastError();
}

}  // namespace moe
