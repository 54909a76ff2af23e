/*
 * moe.h -- C ABI of the expert-grouped, group-quantized MoE layer for MI355X.
 *
 * The layer (pages on serving Qwen3.8-Flash-Next):
 *   - TandemLLM docs, chapter 17 "Qwen3.8-Flash-Next", Table 17.1: 512 routed
 *     experts a layer; every token runs 10 of them plus 1 shared expert.
 *   - "Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated prefill lane"
 *     (its numbered list): the grouped lane this library implements.
 *     moe_permute orders every (token, slot) assignment by expert on the GPU,
 *     identically on every run; moe_grouped_ffn runs each expert's SwiGLU
 *     once over all of its rows (quantized weights, 16-bit activations),
 *     scales the intermediate by the token's routing weight before the down
 *     projection, and keeps each assignment's result as its own fp32 row;
 *     moe_combine adds a token's rows in slot order, so nothing accumulates
 *     through atomics.
 *   - same README, section "Independent decode lane": the 512-expert router
 *     uses a deterministic stable top-k (moe_route).
 *   - same README, "Model artifact and memory placement" table: routed experts
 *     stored as symmetric grouped int4/int8, the router kept unquantized.
 *   - TandemLLM roadmap, "A mixture-of-experts model, and what is left", and
 *     chapter 17, section 17.2: expert packs coded at other bit widths, MoE
 *     kernels that take 2 to 6 and 8 bits (here 2, 3, 5, 6, 7 and 8-bit
 *     group-32 codes beside int4).
 *   - "anvil-serving" benchmark dossier, Qwen3.8-Flash-Next entry, section
 *     "Quantization boundary": W4A4 (4-bit weights and activations) on the
 *     routed experts only, the shared expert kept 16-bit.  Here in the OCP
 *     Microscaling FP4 format that CDNA4's scaled MFMA takes (MOE_MXFP4).
 *
 * Conventions for every call below:
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates device memory; what a call leaves behind lives in the
 *     caller's buffers (moe_route_plan's counters in the workspace, zero
 *     between calls), apart from moe_grouped_ffn_noalloc's static scratch.
 *   - Device calls (moe_route*, moe_permute, moe_grouped_ffn, moe_combine)
 *     take device pointers and a hipStream_t passed as `void* stream` (NULL =
 *     the null stream).  They only enqueue work: nothing synchronizes, so a
 *     layer's calls can be captured in one HIP graph.  They run on the device
 *     current to the calling thread.
 *   - Errors: arguments are checked on the host before anything is enqueued.
 *     A failed check returns a negative moe_status and sets a thread-local
 *     message (moe_last_error).  A launch failure returns MOE_EDEVICE.  T == 0
 *     returns MOE_OK and enqueues nothing.  Values inside device buffers (for
 *     example expert ids) are preconditions and are not checked.
 *   - Alignment: every device pointer must be 16-byte aligned; the workspace
 *     256-byte aligned.
 *   - Reentrancy: calls are thread-safe; concurrent calls need distinct
 *     workspaces and outputs.
 *
 * Canonical weight layouts (what moe_pack_experts reads), per expert, experts
 * stacked contiguously:
 *   gate [F, d], up [F, d], down [d, F]   row-major, K (the reduced dim) last.
 *   MOE_F32 / MOE_BF16: one element per weight.
 *   MOE_I4_G32: symmetric int4, two's complement, codes in [-7, 7]; byte j of a
 *     row holds element 2j in its low nibble and 2j+1 in its high nibble; one
 *     fp16 scale per 32 consecutive elements along K, scales [rows, K/32].
 *     Weight value = code * scale.
 *   MOE_I8_ROW: int8 codes in [-127, 127], one fp16 scale per row, scales [rows].
 *   MOE_I2_G32 .. MOE_I8_G32 (b = 2, 3, 5, 6, 7, 8 bits): symmetric b-bit codes
 *     in [-(2^(b-1) - 1), 2^(b-1) - 1], one int8 per code, [rows, K]; one fp16
 *     scale per 32 consecutive elements along K, scales [rows, K/32].  Weight
 *     value = code * scale.  The device blob stores them at b bits per weight
 *     (plus the scales).
 *   MOE_MXFP4: OCP MX FP4 (e2m1) codes, byte j of a row holds element 2j in its
 *     low nibble, [rows, K/2]; one E8M0 scale byte per 32 consecutive elements
 *     along K, scales [rows, K/32] (uint8).  Weight value = e2m1(code) *
 *     2^(scale - 127); e2m1 is sign bit 3, exponent bits 2..1 (bias 1),
 *     mantissa bit 0, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  A scale byte of
 *     255 (NaN) is rejected by the packer.
 * The device blob written by moe_pack_experts is a private, tile-ordered
 * layout; its only contract is moe_pack_experts / moe_unpack_experts.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument: null pointer, bad size, misalignment */
  MOE_EUNSUPPORTED = -2, /* valid request that this library does not implement */
  MOE_EWORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes()        */
  MOE_EDEVICE = -4       /* the HIP runtime reported an error                   */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,    /* IEEE binary32                                     */
  MOE_BF16 = 1,   /* bfloat16                                          */
  MOE_I4_G32 = 2, /* symmetric int4 + fp16 scale per 32 along K        */
  MOE_I8_ROW = 3, /* symmetric int8 + fp16 scale per output row        */
  MOE_I2_G32 = 4, /* symmetric b-bit codes + fp16 scale per 32 along K  */
  MOE_I3_G32 = 5,
  MOE_I5_G32 = 6,
  MOE_I6_G32 = 7,
  MOE_I7_G32 = 8,
  MOE_I8_G32 = 9,
  MOE_MXFP4 = 10  /* OCP MX FP4: e2m1 codes + E8M0 scale per 32 along K (W4A4) */
} moe_dtype;

typedef enum moe_blob_kind {
  MOE_BLOB_ROUTED = 0, /* the n_experts routed experts */
  MOE_BLOB_SHARED = 1  /* the shared expert            */
} moe_blob_kind;

/* Shape and storage of one MoE layer.
 * Supported combinations:
 *   act MOE_F32 : expert_w MOE_F32, shared_w MOE_F32 (router fp32, y fp32)
 *   act MOE_BF16: expert_w MOE_BF16, MOE_I4_G32, MOE_I{2,3,5,6,7,8}_G32 or
 *                 MOE_MXFP4, shared_w MOE_BF16 or MOE_I8_ROW  (router bf16,
 *                 y bf16)
 * Sizes: 1 <= n_experts <= 1024; n_shared 0 or 1; every call needs
 * T*k <= 2^30 and T*k*max(ffn, shared_ffn), T*d < 2^31.  For act MOE_BF16:
 * d % 256 == 0, ffn % 128 == 0 (% 256 with 2- or 4-bit or MXFP4 routed
 * weights), shared_ffn % 128 == 0.  For act MOE_F32:
 * d, ffn, shared_ffn multiples of 64.  d, ffn, shared_ffn <= 16384.         */
typedef struct moe_desc {
  int32_t d;          /* hidden width                                       */
  int32_t n_experts;  /* E, routed experts                                  */
  int32_t ffn;        /* F, SwiGLU width of a routed expert                 */
  int32_t n_shared;   /* 0 or 1 always-active shared expert                 */
  int32_t shared_ffn; /* Fs, SwiGLU width of the shared expert (0 if none)  */
  int32_t act;        /* moe_dtype of hidden, router weights and y          */
  int32_t expert_w;   /* moe_dtype of the routed expert weights             */
  int32_t shared_w;   /* moe_dtype of the shared expert weights             */
} moe_desc;

/* ---------------------------------------------------------------- host only */

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

/* Static text for a status code ("ok", "invalid argument", ...). */
const char* moe_status_str(int32_t status);

/* Thread-local text describing the last failed call on this thread ("" if
 * none).  Valid until the next library call on the same thread.            */
const char* moe_last_error(void);

/* Bytes of the device blob that holds the routed experts (kind ROUTED) or the
 * shared expert (kind SHARED) of `desc`: the expert packs of the
 * "Qwen3.8-Flash-Next-Dual-GPU" README, "Model artifact and memory
 * placement" table (routed experts as grouped int4/int8 codes beside their
 * scales, resident on the GPU).  Host only, no GPU touched.                 */
moe_status moe_blob_bytes(const moe_desc* desc, int32_t kind, size_t* bytes);

/* Pack canonical weights (layouts above; `*_scales` NULL for F32/BF16) into
 * the private device blob (the expert packs of the same README table; the
 * b-bit codes of the TandemLLM roadmap's "A mixture-of-experts model, and
 * what is left"), written to the host buffer `blob` of `blob_bytes`
 * (>= moe_blob_bytes).  The caller copies it to device memory.  For ROUTED the
 * inputs hold n_experts experts stacked; for SHARED one expert.
 * MOE_I4_G32 codes must lie in [-7, 7] (symmetric); an 8 (-8) code returns
 * MOE_EINVAL, as does a b-bit code outside [-(2^(b-1) - 1), 2^(b-1) - 1] and
 * an MXFP4 scale byte of 255.  fp16 scales must be finite; a group scale of
 * the int4 or b-bit formats must also keep its largest product finite in
 * fp16, |scale| * (2^(b-1) - 1) < 65520 (|scale| <= 9352 for int4), because
 * the gate/up products take fp16(code * scale) as their weights; any other
 * scale returns MOE_EINVAL.  Scales below fp16's normal range are fine: a
 * code times such a scale is exact or rounded at fp16 precision.
 * Host only.                                                                */
moe_status moe_pack_experts(const moe_desc* desc, int32_t kind, const void* gate,
                            const void* gate_scales, const void* up, const void* up_scales,
                            const void* down, const void* down_scales, void* blob,
                            size_t blob_bytes);

/* Inverse of moe_pack_experts: canonical weights from a host copy of a blob
 * (outputs sized as the canonical inputs; `*_scales` ignored for F32/BF16). */
moe_status moe_unpack_experts(const moe_desc* desc, int32_t kind, const void* blob,
                              size_t blob_bytes, void* gate, void* gate_scales, void* up,
                              void* up_scales, void* down, void* down_scales);

/* Bytes of device workspace that moe_permute, moe_route_plan and
 * moe_grouped_ffn need for T tokens and top-k (the route plan and the
 * intermediate h of the README's "Dedicated prefill lane", steps 1-3).  Nothing in it needs
 * initializing, except the first 16 bytes for moe_route_plan (zero; see
 * there).  Host only.                                                      */
moe_status moe_workspace_bytes(const moe_desc* desc, int32_t T, int32_t k, size_t* bytes);

/* ------------------------------------------------------------------ device */

/* Router and stable top-k ("Independent decode lane").
 *   hidden    [T, d]  act dtype, row-major
 *   router_w  [E, d]  act dtype, row-major (never quantized)
 *   bias      [E] fp32 added to every logit, or NULL
 *   logits    [T, E] fp32 out: sum_i hidden[t,i]*router_w[e,i] (+ bias[e]),
 *             accumulated in fp32
 *   topk_ids  [T, k] int32 out: per token the k experts in order of (logit
 *             descending, expert id ascending); -0.0 ties +0.0
 *   topk_w    [T, k] fp32 out: softmax over the k chosen logits
 * 1 <= k <= min(E, 32).  Logits must be finite (NaN/Inf order is undefined). */
moe_status moe_route(const moe_desc* desc, int32_t T, int32_t k, const void* hidden,
                     const void* router_w, const float* bias, float* logits, int32_t* topk_ids,
                     float* topk_w, void* stream);

/* The top-k and softmax of moe_route alone, on caller-given fp32 logits
 * [T, E] (same outputs and rules as moe_route).                             */
moe_status moe_route_from_logits(const moe_desc* desc, int32_t T, int32_t k, const float* logits,
                                 int32_t* topk_ids, float* topk_w, void* stream);

/* Route plan ("Dedicated prefill lane", step 1): the assignments ordered by
 * expert, the same order on every run.
 *   hidden    [T, d] act dtype, the layer's input (read only by int4 and b-bit
 *             layers: see workspace)
 *   topk_ids  [T*k] int32, flat index f = t*k + s, values in [0, E)
 *   offsets   [E+1] int32 out: offsets[e] = #{f : ids[f] < e}; offsets[E] = T*k
 *   perm      [T*k] int32 out: the f of expert e, ascending, at
 *             perm[offsets[e] .. offsets[e+1])
 *   inv_perm  [T*k] int32 out: inv_perm[perm[p]] = p
 *   workspace scratch of >= moe_workspace_bytes(desc, T, k); this call also
 *             leaves in it what moe_grouped_ffn reads besides its arguments --
 *             the row-tile plan, and for int4 / b-bit layers the fp16 copy
 *             of hidden that their gate/up products run on (each token row
 *             scaled by a power of two) -- so pass the same workspace, unchanged,
 *             and the same hidden to the moe_grouped_ffn call that consumes
 *             this plan.                                                   */
moe_status moe_permute(const moe_desc* desc, int32_t T, int32_t k, const void* hidden,
                       const int32_t* topk_ids, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, void* workspace, size_t workspace_bytes,
                       void* stream);

/* moe_route followed by moe_permute, as one call: the same arguments, the
 * same outputs bit for bit (logits, topk_ids, topk_w, offsets, perm,
 * inv_perm, and in the workspace the row-tile plan and the fp16 copy of
 * hidden that moe_grouped_ffn reads).  For a small call -- act BF16 and
 * T <= 32, where launches and latency rather than bytes set the time --
 * it is a single kernel launch (TandemLLM Roadmap v0.11.2, "Parallel
 * requests": a joint pass of up to 32 rows should cost about what its bytes
 * cost); otherwise it issues moe_route's and moe_permute's launches.
 *   workspace  >= moe_workspace_bytes(desc, T, k).  Its first 16 bytes
 *              hold the single launch's block counters: they must be zero
 *              before the first moe_route_plan call on this workspace (zero
 *              them once after allocating it); every call leaves them zero,
 *              and no other call writes them.  Calls that share a workspace
 *              must be ordered (one stream), as for moe_permute.
 * Errors as moe_route and moe_permute.                                    */
moe_status moe_route_plan(const moe_desc* desc, int32_t T, int32_t k, const void* hidden,
                          const void* router_w, const float* bias, float* logits,
                          int32_t* topk_ids, float* topk_w, int32_t* offsets, int32_t* perm,
                          int32_t* inv_perm, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Expert-grouped SwiGLU ("Dedicated prefill lane", steps 2-4).  For each
 * expert e and each p in [offsets[e], offsets[e+1]), with f = perm[p],
 * t = f / k and weight w = topk_w[f]:
 *   h = w * silu(Wg_e x_t) (.) (Wu_e x_t)        (router weight folded in)
 *   out_assign[p] = Wd_e h                       fp32, one row per assignment
 * and for the shared expert (n_shared == 1), every token t:
 *   shared_out[t] = Wd_s (silu(Wg_s x_t) (.) (Wu_s x_t))   fp32
 *   hidden      [T, d] act dtype
 *   topk_w      [T*k] fp32 (from moe_route)
 *   offsets, perm        from moe_permute
 *   routed_blob, shared_blob  device copies of moe_pack_experts blobs
 *             (shared_blob NULL iff n_shared == 0)
 *   out_assign  [T*k, d] fp32 out, in permuted order (row p)
 *   shared_out  [T, d] fp32 out (NULL iff n_shared == 0)
 *   workspace   the workspace moe_permute filled (holds its tile plan and the
 *               intermediate h).
 * Arithmetic (act BF16): MFMA with fp32 accumulation.  bf16 weights run bf16
 * MFMA.  With int4 (or other b-bit group-32) routed weights the gate/up
 * products run fp16 MFMA on an fp16 copy of x, each token row scaled by a
 * power of two so its largest magnitude lies in [2^14, 2^15) (undone on the
 * fp32 accumulator); the codes become fp16(code * scale) there and
 * bf16(code * scale) in the down product; int8 codes enter exactly, their row
 * scale applied to the
 * fp32 accumulator.  h is rounded to bf16 (nearest even); the outputs stay
 * fp32.  The fp32 path computes and stores in fp32 throughout.
 * MOE_MXFP4 routed experts run W4A4 on the scaled FP4 MFMA: each token row of
 * hidden is quantized to MXFP4 block by block of 32 (OCP MX rule: shared
 * exponent E = floor(log2 max|v|) - 2, clamped to [-127, 127], -127 for an
 * all-zero block; element = nearest e2m1 value of v / 2^E, ties to even,
 * saturated at +-6), the gate/up products and h = w * silu(g) * u are
 * computed in fp32, h is quantized the same way per row and 32 columns
 * (straight from fp32), and the down product runs on those codes; fp32
 * accumulation throughout.  The shared expert of such a layer runs on the
 * unquantized bf16 hidden rows (bf16 MFMA).                                */
moe_status moe_grouped_ffn(const moe_desc* desc, int32_t T, int32_t k, const void* hidden,
                           const float* topk_w, const int32_t* offsets, const int32_t* perm,
                           const void* routed_blob, const void* shared_blob, float* out_assign,
                           float* shared_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* moe_grouped_ffn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs and arithmetic as moe_grouped_ffn, minus the
 * workspace: the row-tile plan is rebuilt from `offsets` (so moe_permute's
 * plan in a workspace is not needed) and every intermediate lives in a
 * scratch array of 8 MiB that the library keeps on each GPU it runs on until
 * the process ends.  A call whose moe_workspace_bytes(desc, T, k) exceeds
 * 8 MiB returns MOE_EWORKSPACE and enqueues nothing (d=2560, ffn=1024,
 * k=10, int4 routed and int8 shared experts: up to T = 302).  The first
 * call on a GPU looks up that GPU's scratch address (hipGetSymbolAddress; no
 * allocation).  Calls that overlap on one GPU -- from two streams or two
 * threads -- share the scratch and race: the caller must order them.       */
moe_status moe_grouped_ffn_noalloc(const moe_desc* desc, int32_t T, int32_t k, const void* hidden,
                                   const float* topk_w, const int32_t* offsets,
                                   const int32_t* perm, const void* routed_blob,
                                   const void* shared_blob, float* out_assign, float* shared_out,
                                   void* stream);

/* Fixed-order combine ("Dedicated prefill lane", step 5), no atomics:
 *   y[t] = act( ((out_assign[inv_perm[t*k+0]] + ... ) + out_assign[inv_perm[t*k+k-1]])
 *               + shared_out[t] )
 * summed in fp32 in exactly that order, then rounded to the act dtype (bf16:
 * round to nearest even).  shared_out may be NULL (n_shared == 0).
 *   y [T, d] act dtype out.                                                 */
moe_status moe_combine(const moe_desc* desc, int32_t T, int32_t k, const float* out_assign,
                       const int32_t* inv_perm, const float* shared_out, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
