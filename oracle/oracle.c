/*
 * oracle.c -- plain, slow, fp64 CPU reference of the expert-grouped MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg do.  It shares no code, header or table with
 * the HIP library and includes nothing from it.
 *
 * What it follows (the web pages on serving Qwen3.8-Flash-Next):
 *   - "Qwen3.8-Flash-Next" (TandemLLM docs, chapter 17), Table 17.1: each
 *     token runs 10 routed experts out of 512 plus 1 shared expert.
 *   - "Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated prefill lane"
 *     (its numbered list): assignments grouped by expert in a reproducible
 *     order, each expert's matrices applied to its group, the routing weight
 *     applied to the intermediate before the down projection, a separate
 *     result per assignment, and each token's results added in slot order.
 *   - same README, section "Independent decode lane": the 512-expert router
 *     uses a deterministic stable top-k.
 *   - same README, "Model artifact and memory placement" table: symmetric
 *     group-quantized expert weights; the router is never quantized.
 *
 * Readings where the pages leave a step open (all fp64 here):
 *   - router logit = sum_i x[i] * Wr[e][i] (+ bias[e] when a bias is given);
 *   - top-k order: larger logit first, equal logits -> lower expert id first;
 *     slot s is rank s;
 *   - routing weights: softmax over the k chosen logits only;
 *   - expert: Wd * (silu(Wg x) (.) Wu x), silu(a) = a / (1 + exp(-a)),
 *     no biases; the shared expert has no gate and weight 1;
 *   - route plan: stable counting sort of flat index f = t*k + s by expert;
 *   - int4: two's complement nibbles, element 2j in the low nibble, value
 *     q * s with one fp16 scale per 32 consecutive elements along K;
 *     int8: value q * s with one fp16 scale per output row;
 *     b-bit codes (b = 2, 3, 5, 6, 7, 8; TandemLLM roadmap, "A mixture-of-
 *     experts model, and what is left", and chapter 17, section 17.2: expert
 *     packs at other bit widths): one int8 per code, symmetric range
 *     [-(2^(b-1) - 1), 2^(b-1) - 1], value q * s with one fp16 scale per 32
 *     consecutive elements along K.
 *   - MXFP4 W4A4 routed experts (the analog, in the OCP Microscaling (MX)
 *     formats, of the NVFP4 W4A4 routed experts of the "anvil-serving"
 *     dossier, section "Quantization boundary"): weights are e2m1 codes with
 *     one E8M0 power-of-two scale per 32 along K; the expert's two inputs --
 *     the token row x and the folded intermediate h = w * silu(g) * u -- are
 *     quantized to MXFP4 the same way (OCP MX rule, orc_mx_quantize) before
 *     the products; the shared expert stays on the unquantized x.
 *
 * Every arithmetic step runs in double precision on the exact upcast of the
 * stored values.  There is no blocking, fusion or reordering: each function
 * is the definition written out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0   /* IEEE binary32                                   */
#define ORC_BF16 1  /* bfloat16 bit patterns (uint16)                   */
#define ORC_I4G32 2 /* int4 two's complement + fp16 scale per 32 along K */
#define ORC_I8ROW 3 /* int8 + fp16 scale per row                        */
#define ORC_MXFP4 4 /* e2m1 nibbles + E8M0 scale byte per 32 along K   */
#define ORC_IG32 16 /* + b: b-bit codes (one int8 each) + fp16 scale per 32 along K */
static int ig32_bits(int fmt) {
  const int b = fmt - ORC_IG32;
  return (b >= 2 && b <= 8 && b != 4) ? b : 0;
}

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ENOMEM -2
#define ORC_ENONFINITE -3

/* ---- scalar decoders --------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return sign ? -v : v;
}

/* OCP MX e2m1 (FP4): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 * mantissa; exponent 0 is subnormal, m * 2^-1.                             */
double orc_e2m1_to_f64(int code) {
  const int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -v : v;
}

/* OCP MX E8M0 scale: 2^(s - 127); s = 255 is NaN.                          */
double orc_e8m0_to_f64(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* signed value of nibble j of a row of packed int4 (low nibble = even j) */
static int nibble_value(const uint8_t* row, int64_t j) {
  uint8_t byte = row[j / 2];
  int n = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
  return n >= 8 ? n - 16 : n;
}

/* Decode a stored [rows, K] matrix to doubles.
 *   F32 : q = float[rows*K]
 *   BF16: q = uint16[rows*K]
 *   I4G32: q = uint8[rows*K/2], scales = uint16 (fp16) [rows*K/32]
 *   I8ROW: q = int8[rows*K],    scales = uint16 (fp16) [rows]
 *   IG32+b: q = int8[rows*K],   scales = uint16 (fp16) [rows*K/32]; a code
 *           outside [-(2^(b-1) - 1), 2^(b-1) - 1] is an error
 *   MXFP4: q = uint8[rows*K/2] e2m1 nibbles (low nibble = even j),
 *          scales = uint8 E8M0 [rows*K/32]; a NaN scale (255) is an error  */
int orc_decode_matrix(int fmt, int64_t rows, int64_t K, const void* q, const void* scales,
                      double* out) {
  if (rows < 0 || K < 0 || (rows * K > 0 && (!q || !out))) return ORC_EINVAL;
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t j = 0; j < K; j++) {
      double v;
      if (fmt == ORC_F32) {
        v = (double)((const float*)q)[r * K + j];
      } else if (fmt == ORC_BF16) {
        v = orc_bf16_to_f64(((const uint16_t*)q)[r * K + j]);
      } else if (fmt == ORC_I4G32) {
        if (K % 32 != 0 || !scales) return ORC_EINVAL;
        const uint8_t* row = (const uint8_t*)q + r * (K / 2);
        double s = orc_f16_to_f64(((const uint16_t*)scales)[r * (K / 32) + j / 32]);
        v = (double)nibble_value(row, j) * s;
      } else if (fmt == ORC_I8ROW) {
        if (!scales) return ORC_EINVAL;
        double s = orc_f16_to_f64(((const uint16_t*)scales)[r]);
        v = (double)((const int8_t*)q)[r * K + j] * s;
      } else if (fmt == ORC_MXFP4) {
        if (K % 32 != 0 || !scales) return ORC_EINVAL;
        const uint8_t byte = ((const uint8_t*)q)[r * (K / 2) + j / 2];
        const uint8_t sc = ((const uint8_t*)scales)[r * (K / 32) + j / 32];
        if (sc == 255) return ORC_EINVAL;
        v = orc_e2m1_to_f64(j % 2 == 0 ? (byte & 15) : (byte >> 4)) * orc_e8m0_to_f64(sc);
      } else if (ig32_bits(fmt)) {
        if (K % 32 != 0 || !scales) return ORC_EINVAL;
        const int lim = (1 << (ig32_bits(fmt) - 1)) - 1;
        const int c = ((const int8_t*)q)[r * K + j];
        if (c < -lim || c > lim) return ORC_EINVAL;
        double s = orc_f16_to_f64(((const uint16_t*)scales)[r * (K / 32) + j / 32]);
        v = (double)c * s;
      } else {
        return ORC_EINVAL;
      }
      out[r * K + j] = v;
    }
  }
  return ORC_OK;
}

/* bytes used by one stored [rows, K] matrix and its scales */
static int64_t q_bytes(int fmt, int64_t rows, int64_t K) {
  switch (fmt) {
    case ORC_F32: return rows * K * 4;
    case ORC_BF16: return rows * K * 2;
    case ORC_I4G32: return rows * K / 2;
    case ORC_I8ROW: return rows * K;
    case ORC_MXFP4: return rows * K / 2;
  }
  if (ig32_bits(fmt)) return rows * K;
  return -1;
}
static int64_t s_bytes(int fmt, int64_t rows, int64_t K) {
  if (fmt == ORC_I4G32 || ig32_bits(fmt)) return rows * (K / 32) * 2;
  if (fmt == ORC_I8ROW) return rows * 2;
  if (fmt == ORC_MXFP4) return rows * (K / 32);
  return 0;
}

/* ---- OCP MX quantization (MXFP4) ----------------------------------------- */

/* The e2m1 value nearest y, ties to the even mantissa, saturated at +-6.
 * The e2m1 magnitudes are 0, 0.5, 1, 1.5 (spacing 0.5 below 2), 2, 3
 * (spacing 1 below 4) and 4, 6 (spacing 2): rounding y / spacing to the
 * nearest integer, ties to even, is rounding to the even mantissa.         */
double orc_e2m1_round(double y) {
  const double a = fabs(y);
  const double step = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
  double q = nearbyint(a / step) * step;
  if (q > 6.0) q = 6.0;
  return y < 0 ? -q : q;
}

/* Shared exponent of one MX block: floor(log2 amax) - 2 (2 is the largest
 * e2m1 exponent), clamped to the E8M0 range [-127, 127]; -127 for amax 0. */
int orc_mx_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int ex;
  frexp(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1 */
  int E = ex - 1 - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

/* OCP MX quantization of v[0..n) (n % 32 == 0), block by block of 32:
 * out[i] = e2m1_round(v[i] / 2^E) * 2^E with E the block's shared exponent;
 * ebits[b] = E + 127 (the E8M0 byte) when ebits is not NULL.               */
int orc_mx_quantize(int64_t n, const double* v, double* out, uint8_t* ebits) {
  if (n < 0 || n % 32 != 0) return ORC_EINVAL;
  for (int64_t b = 0; b < n / 32; b++) {
    double amax = 0.0;
    for (int64_t i = 32 * b; i < 32 * b + 32; i++)
      if (fabs(v[i]) > amax) amax = fabs(v[i]);
    const int E = orc_mx_exponent(amax);
    for (int64_t i = 32 * b; i < 32 * b + 32; i++)
      out[i] = ldexp(orc_e2m1_round(ldexp(v[i], -E)), E);
    if (ebits) ebits[b] = (uint8_t)(E + 127);
  }
  return ORC_OK;
}

/* ---- router ------------------------------------------------------------ */

/* logits[r][e] = sum_i x[tok[r]][i] * Wr[e][i] (+ bias[e])                 */
int orc_router_logits(int64_t n_rows, const int64_t* tok, int64_t d, int64_t E, int x_fmt,
                      const void* x, int wr_fmt, const void* wr, const float* bias,
                      double* logits) {
  double* wrd = (double*)malloc(sizeof(double) * (size_t)(E * d));
  double* xr = (double*)malloc(sizeof(double) * (size_t)d);
  if (!wrd || !xr) { free(wrd); free(xr); return ORC_ENOMEM; }
  free(xr);
  int rc = orc_decode_matrix(wr_fmt, E, d, wr, NULL, wrd);
  if (rc != ORC_OK) { free(wrd); return rc; }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; r++) {
    double* xrow = (double*)malloc(sizeof(double) * (size_t)d);
    int64_t t = tok ? tok[r] : r;
    if (!xrow || orc_decode_matrix(x_fmt, 1, d, (const char*)x + t * q_bytes(x_fmt, 1, d), NULL,
                                   xrow) != ORC_OK) {
#pragma omp atomic write
      rc = ORC_ENOMEM;
      free(xrow);
      continue;
    }
    for (int64_t e = 0; e < E; e++) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; i++) acc += xrow[i] * wrd[e * d + i];
      logits[r * E + e] = acc + (bias ? (double)bias[e] : 0.0);
    }
    free(xrow);
  }
  free(wrd);
  return rc;
}

/* ---- stable top-k and softmax over the chosen k ------------------------ */

/* For each row: pick k experts in order of (logit descending, id ascending);
 * slot s holds the rank-s expert; w[s] = exp(l_s - l_0) / sum_j exp(l_j - l_0)
 * over the chosen j.  Logits must be finite.  -0.0 and +0.0 compare equal. */
int orc_topk_softmax(int64_t n_rows, int64_t E, int64_t k, const double* logits, int32_t* ids,
                     double* w) {
  if (k < 1 || k > E) return ORC_EINVAL;
  char* taken = (char*)malloc((size_t)E);
  if (!taken) return ORC_ENOMEM;
  int rc = ORC_OK;
  for (int64_t r = 0; r < n_rows && rc == ORC_OK; r++) {
    const double* l = logits + r * E;
    for (int64_t e = 0; e < E; e++) {
      if (!isfinite(l[e])) rc = ORC_ENONFINITE;
      taken[e] = 0;
    }
    if (rc != ORC_OK) break;
    for (int64_t s = 0; s < k; s++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++) {
        if (taken[e]) continue;
        /* strictly greater wins; an equal logit never displaces a lower id */
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[r * k + s] = (int32_t)best;
    }
    double l0 = l[ids[r * k]];
    double sum = 0.0;
    for (int64_t s = 0; s < k; s++) sum += exp(l[ids[r * k + s]] - l0);
    for (int64_t s = 0; s < k; s++) w[r * k + s] = exp(l[ids[r * k + s]] - l0) / sum;
  }
  free(taken);
  return rc;
}

/* ---- expert-major route plan -------------------------------------------- */

/* counts[e] = #{f : ids[f] == e}; offsets = exclusive prefix sum (E+1
 * entries, offsets[E] = n); perm = stable counting sort of f by ids[f]
 * (ascending f inside each expert); inv_perm[perm[p]] = p.                 */
int orc_route_plan(int64_t n, int64_t E, const int32_t* ids, int32_t* offsets, int32_t* perm,
                   int32_t* inv_perm) {
  int64_t* cursor = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  if (!cursor) return ORC_ENOMEM;
  for (int64_t f = 0; f < n; f++) {
    if (ids[f] < 0 || ids[f] >= E) { free(cursor); return ORC_EINVAL; }
    cursor[ids[f] + 1]++;
  }
  for (int64_t e = 0; e < E; e++) cursor[e + 1] += cursor[e];
  for (int64_t e = 0; e <= E; e++) offsets[e] = (int32_t)cursor[e];
  for (int64_t f = 0; f < n; f++) {
    int64_t p = cursor[ids[f]]++;
    perm[p] = (int32_t)f;
    inv_perm[f] = (int32_t)p;
  }
  free(cursor);
  return ORC_OK;
}

/* ---- one SwiGLU expert on one row ---------------------------------------- */

static double silu(double a) { return a / (1.0 + exp(-a)); }

/* out[0..d) = Wd * (silu(Wg x) (.) (Wu x));  Wg, Wu: [F, d], Wd: [d, F]   */
static void swiglu_row(int64_t d, int64_t F, const double* x, const double* wg, const double* wu,
                       const double* wd, double* h, double* out) {
  for (int64_t j = 0; j < F; j++) {
    double g = 0.0, u = 0.0;
    for (int64_t i = 0; i < d; i++) {
      g += wg[j * d + i] * x[i];
      u += wu[j * d + i] * x[i];
    }
    h[j] = silu(g) * u;
  }
  for (int64_t i = 0; i < d; i++) {
    double o = 0.0;
    for (int64_t j = 0; j < F; j++) o += wd[i * F + j] * h[j];
    out[i] = o;
  }
}

/* Decision slack of the MX quantization of h against an h' computed with
 * error: for h' with |h'_j - h_j| <= dh_j, the quantization (a decision on
 * h') may pick the neighbouring code or, through the block maximum, the
 * neighbouring shared exponent.  For F values h (F % 32 == 0):
 *   hq = MX(h);
 *   delta_j  = max |MX(h')_j - hq_j| over that box (the exponents reachable
 *              from the block maximum's range, each end of h_j's interval:
 *              for a fixed exponent the quantization is monotone in h');
 *   slack[i] = sum_j |wd[i][j]| delta_j,  mag[i] = sum_j |wd[i][j] hq_j|
 * for the d rows of wd [d, F].                                             */
int orc_mx_slack(int64_t d, int64_t F, const double* h, const double* dh, const double* wd,
                 double* hq, double* delta, double* slack, double* mag) {
  int rc = orc_mx_quantize(F, h, hq, NULL);
  if (rc != ORC_OK) return rc;
  for (int64_t b = 0; b < F / 32; b++) {
    double lo = 0.0, hi = 0.0;
    for (int64_t j = 32 * b; j < 32 * b + 32; j++) {
      const double a = fabs(h[j]);
      if (a - dh[j] > lo) lo = a - dh[j];
      if (a + dh[j] > hi) hi = a + dh[j];
    }
    const int e_lo = orc_mx_exponent(lo), e_hi = orc_mx_exponent(hi);
    for (int64_t j = 32 * b; j < 32 * b + 32; j++) {
      delta[j] = 0.0;
      const double ends[2] = {h[j] - dh[j], h[j] + dh[j]};
      for (int E = e_lo; E <= e_hi; E++) {
        for (int t = 0; t < 2; t++) {
          const double v = ldexp(orc_e2m1_round(ldexp(ends[t], -E)), E);
          if (fabs(v - hq[j]) > delta[j]) delta[j] = fabs(v - hq[j]);
        }
      }
    }
  }
  for (int64_t i = 0; i < d; i++) {
    double sl = 0.0, m = 0.0;
    for (int64_t j = 0; j < F; j++) {
      sl += fabs(wd[i * F + j]) * delta[j];
      m += fabs(wd[i * F + j] * hq[j]);
    }
    slack[i] = sl;
    mag[i] = m;
  }
  return ORC_OK;
}

/* Bounds on the fp32 arithmetic of a computation checked against the MXFP4
 * W4A4 expert: gamma bounds the error of a dot product relative to the sum
 * of its terms' magnitudes; eta the relative error of the elementwise steps
 * that make h (silu, the products, the folded router weight).             */
typedef struct {
  double gamma, eta;
} orc_mx_err;

/* Routed MXFP4 W4A4 expert on one row, router weight wf folded into h:
 *   xq = MX(x);  g = Wg xq;  u = Wu xq;  h_j = wf * silu(g_j) * u_j;
 *   hq = MX(h);  out = Wd hq        (MX = orc_mx_quantize)
 * work holds d + 4F doubles.  With err given, also slack and mag
 * (orc_mx_slack) for the error box
 *   dh_j = |wf| (1.1 dg (|u| + du) + |silu(g)| du) + eta |h_j|,
 *   dg = gamma sum_i |Wg[j][i] xq_i|, du likewise (1.1 bounds |silu'|).    */
static int swiglu_row_mx(int64_t d, int64_t F, const double* x, const double* wg,
                         const double* wu, const double* wd, double wf, const orc_mx_err* err,
                         double* work, double* out, double* slack, double* mag) {
  double* xq = work;
  double* h = xq + d;
  double* hq = h + F;
  double* dh = hq + F;
  double* delta = dh + F;
  int rc = orc_mx_quantize(d, x, xq, NULL);
  if (rc != ORC_OK) return rc;
  for (int64_t j = 0; j < F; j++) {
    double g = 0.0, u = 0.0, ag = 0.0, au = 0.0;
    for (int64_t i = 0; i < d; i++) {
      g += wg[j * d + i] * xq[i];
      u += wu[j * d + i] * xq[i];
      ag += fabs(wg[j * d + i] * xq[i]);
      au += fabs(wu[j * d + i] * xq[i]);
    }
    h[j] = wf * silu(g) * u;
    if (err) {
      const double dg = err->gamma * ag, du = err->gamma * au;
      dh[j] = fabs(wf) * (1.1 * dg * (fabs(u) + du) + fabs(silu(g)) * du) + err->eta * fabs(h[j]);
    }
  }
  rc = orc_mx_quantize(F, h, hq, NULL);
  if (rc != ORC_OK) return rc;
  for (int64_t i = 0; i < d; i++) {
    double o = 0.0;
    for (int64_t j = 0; j < F; j++) o += wd[i * F + j] * hq[j];
    out[i] = o;
  }
  if (!err) return ORC_OK;
  return orc_mx_slack(d, F, h, dh, wd, hq, delta, slack, mag);
}

/* Dense SwiGLU MLP over M rows with already-decoded weights (used to pin
 * the E=1, k=1 special case against an independent library product). */
int orc_swiglu_dense(int64_t M, int64_t d, int64_t F, const double* X, const double* wg,
                     const double* wu, const double* wd, double* out) {
  double* h = (double*)malloc(sizeof(double) * (size_t)F);
  if (!h) return ORC_ENOMEM;
  for (int64_t m = 0; m < M; m++) swiglu_row(d, F, X + m * d, wg, wu, wd, h, out + m * d);
  free(h);
  return ORC_OK;
}

/* ---- the layer: per-expert loop, shared expert, weighted sum ------------- */

typedef struct {
  int64_t d, E, k, F, n_shared, Fs;
  int x_fmt, expert_fmt, shared_fmt;
} orc_desc;

typedef struct {
  const void* x;                 /* [T, d] stored activations               */
  const void *wg, *wg_s;         /* routed gate [E, F, d] (+ scales)        */
  const void *wu, *wu_s;         /* routed up   [E, F, d] (+ scales)        */
  const void *wd, *wd_s;         /* routed down [E, d, F] (+ scales)        */
  const void *sg, *sg_s;         /* shared gate [Fs, d]   (+ scales)        */
  const void *su, *su_s;         /* shared up   [Fs, d]   (+ scales)        */
  const void *sd, *sd_s;         /* shared down [d, Fs]   (+ scales)        */
} orc_weights;

/* pointer to matrix e of a stacked [E, rows, K] array and its scales */
static const void* mat_q(const void* base, int fmt, int64_t e, int64_t rows, int64_t K) {
  return (const char*)base + e * q_bytes(fmt, rows, K);
}
static const void* mat_s(const void* base, int fmt, int64_t e, int64_t rows, int64_t K) {
  return base ? (const char*)base + e * s_bytes(fmt, rows, K) : NULL;
}

/* For n rows (row r is token tok[r] of x), with routed ids[n*k] and weights
 * w[n*k] (slot order):
 *   out_assign[f]  = w[f] * expert_{ids[f]}(x_t)     (f = r*k + s), [n*k, d]
 *   shared_out[r]  = shared(x_t)                      [n, d] (if n_shared)
 *   y[r]           = sum_{s<k} out_assign[r*k+s] + shared_out[r]
 * The experts run in expert-major order from the route plan, one expert's
 * weights decoded at a time.  out_assign / shared_out may be NULL.          */
static int moe_experts(const orc_desc* D, const orc_weights* W, int64_t n, const int64_t* tok,
                       const int32_t* ids, const double* w, double* out_assign, double* shared_out,
                       double* y, const orc_mx_err* err, double* slack, double* mag) {
  const int64_t d = D->d, E = D->E, k = D->k, F = D->F, Fs = D->Fs, nk = n * k;
  int rc = ORC_OK;
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nk + 1));
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nk + 1));
  double* oa = (double*)malloc(sizeof(double) * (size_t)(nk * d + 1));
  double* so = (double*)calloc((size_t)(n * d + 1), sizeof(double));
  if (!offsets || !perm || !inv || !oa || !so) { rc = ORC_ENOMEM; goto done; }
  rc = orc_route_plan(nk, E, ids, offsets, perm, inv);
  if (rc != ORC_OK) goto done;

  /* routed experts, one expert (and its decoded weights) per iteration */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t e = 0; e < E; e++) {
    if (offsets[e + 1] == offsets[e]) continue;
    double* wg = (double*)malloc(sizeof(double) * (size_t)(F * d));
    double* wu = (double*)malloc(sizeof(double) * (size_t)(F * d));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(d * F));
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* h = (double*)malloc(sizeof(double) * (size_t)(d + 4 * F));
    int lrc = (wg && wu && wd && xr && h) ? ORC_OK : ORC_ENOMEM;
    if (lrc == ORC_OK) lrc = orc_decode_matrix(D->expert_fmt, F, d, mat_q(W->wg, D->expert_fmt, e, F, d), mat_s(W->wg_s, D->expert_fmt, e, F, d), wg);
    if (lrc == ORC_OK) lrc = orc_decode_matrix(D->expert_fmt, F, d, mat_q(W->wu, D->expert_fmt, e, F, d), mat_s(W->wu_s, D->expert_fmt, e, F, d), wu);
    if (lrc == ORC_OK) lrc = orc_decode_matrix(D->expert_fmt, d, F, mat_q(W->wd, D->expert_fmt, e, d, F), mat_s(W->wd_s, D->expert_fmt, e, d, F), wd);
    for (int64_t p = offsets[e]; lrc == ORC_OK && p < offsets[e + 1]; p++) {
      int64_t f = perm[p];
      int64_t t = tok ? tok[f / k] : f / k;
      lrc = orc_decode_matrix(D->x_fmt, 1, d, (const char*)W->x + t * q_bytes(D->x_fmt, 1, d), NULL, xr);
      if (lrc != ORC_OK) break;
      if (D->expert_fmt == ORC_MXFP4) {
        lrc = swiglu_row_mx(d, F, xr, wg, wu, wd, w[f], err, h, oa + f * d,
                            err ? slack + f * d : NULL, err ? mag + f * d : NULL);
      } else {
        swiglu_row(d, F, xr, wg, wu, wd, h, oa + f * d);
        for (int64_t i = 0; i < d; i++) oa[f * d + i] *= w[f];
      }
    }
    if (lrc != ORC_OK) {
#pragma omp atomic write
      rc = lrc;
    }
    free(wg); free(wu); free(wd); free(xr); free(h);
  }
  if (rc != ORC_OK) goto done;

  /* shared expert: every row, weight 1 */
  if (D->n_shared) {
    double* sg = (double*)malloc(sizeof(double) * (size_t)(Fs * d));
    double* su = (double*)malloc(sizeof(double) * (size_t)(Fs * d));
    double* sd = (double*)malloc(sizeof(double) * (size_t)(d * Fs));
    if (!sg || !su || !sd) rc = ORC_ENOMEM;
    if (rc == ORC_OK) rc = orc_decode_matrix(D->shared_fmt, Fs, d, W->sg, W->sg_s, sg);
    if (rc == ORC_OK) rc = orc_decode_matrix(D->shared_fmt, Fs, d, W->su, W->su_s, su);
    if (rc == ORC_OK) rc = orc_decode_matrix(D->shared_fmt, d, Fs, W->sd, W->sd_s, sd);
    if (rc == ORC_OK) {
#pragma omp parallel for schedule(dynamic, 1)
      for (int64_t r = 0; r < n; r++) {
        double* xr = (double*)malloc(sizeof(double) * (size_t)d);
        double* h = (double*)malloc(sizeof(double) * (size_t)Fs);
        int64_t t = tok ? tok[r] : r;
        if (xr && h &&
            orc_decode_matrix(D->x_fmt, 1, d, (const char*)W->x + t * q_bytes(D->x_fmt, 1, d), NULL, xr) == ORC_OK)
          swiglu_row(d, Fs, xr, sg, su, sd, h, so + r * d);
        else {
#pragma omp atomic write
          rc = ORC_ENOMEM;
        }
        free(xr); free(h);
      }
    }
    free(sg); free(su); free(sd);
    if (rc != ORC_OK) goto done;
  }

  /* weighted sum: slots 0..k-1 in order, then the shared expert */
  for (int64_t r = 0; r < n; r++) {
    for (int64_t i = 0; i < d; i++) {
      double acc = 0.0;
      for (int64_t s = 0; s < k; s++) acc += oa[(r * k + s) * d + i];
      y[r * d + i] = acc + so[r * d + i];
    }
  }
  if (out_assign) memcpy(out_assign, oa, sizeof(double) * (size_t)(nk * d));
  if (shared_out) memcpy(shared_out, so, sizeof(double) * (size_t)(n * d));
done:
  free(offsets); free(perm); free(inv); free(oa); free(so);
  return rc;
}

int orc_moe_experts(const orc_desc* D, const orc_weights* W, int64_t n, const int64_t* tok,
                    const int32_t* ids, const double* w, double* out_assign, double* shared_out,
                    double* y) {
  return moe_experts(D, W, n, tok, ids, w, out_assign, shared_out, y, NULL, NULL, NULL);
}

/* The layer as orc_moe_experts, plus, for MXFP4 routed experts, mag and
 * slack (swiglu_row_mx) of every assignment row f = r*k + s, [n*k, d].    */
int orc_moe_experts_mx(const orc_desc* D, const orc_weights* W, int64_t n, const int64_t* tok,
                       const int32_t* ids, const double* w, double gamma, double eta,
                       double* out_assign, double* shared_out, double* y, double* slack,
                       double* mag) {
  if (D->expert_fmt != ORC_MXFP4 || !slack || !mag) return ORC_EINVAL;
  const orc_mx_err err = {gamma, eta};
  return moe_experts(D, W, n, tok, ids, w, out_assign, shared_out, y, &err, slack, mag);
}
