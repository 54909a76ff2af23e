// abi.cpp -- the C ABI of include/moe.h: argument checks (host only, before
// anything is enqueued), the blob packer, workspace sizing and launch dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <thread>
#include <vector>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_desc(const moe_desc* D) {
  if (!D) return fail(MOE_EINVAL, "desc is NULL");
  if (D->n_experts < 1 || D->n_experts > MAX_EXPERTS)
    return fail(MOE_EINVAL, "n_experts=%d outside [1, %d]", D->n_experts, MAX_EXPERTS);
  if (D->n_shared != 0 && D->n_shared != 1)
    return fail(MOE_EINVAL, "n_shared=%d must be 0 or 1", D->n_shared);
  if (D->d < 1 || D->d > 16384 || D->ffn < 1 || D->ffn > 16384)
    return fail(MOE_EINVAL, "d=%d / ffn=%d outside [1, 16384]", D->d, D->ffn);
  if (D->n_shared && (D->shared_ffn < 1 || D->shared_ffn > 16384))
    return fail(MOE_EINVAL, "shared_ffn=%d outside [1, 16384]", D->shared_ffn);
  if (D->act == MOE_F32) {
    if (D->expert_w != MOE_F32 || (D->n_shared && D->shared_w != MOE_F32))
      return fail(MOE_EUNSUPPORTED, "act F32 needs F32 routed and shared weights");
    if (D->d % 64 || D->ffn % 64 || (D->n_shared && D->shared_ffn % 64))
      return fail(MOE_EUNSUPPORTED, "F32 path needs d, ffn, shared_ffn multiples of 64");
  } else if (D->act == MOE_BF16) {
    if (D->expert_w != MOE_BF16 && ig32_bits(D->expert_w) == 0 && D->expert_w != MOE_MXFP4)
      return fail(MOE_EUNSUPPORTED,
                  "act BF16 needs routed weights BF16, I4_G32, I{2,3,5,6,7,8}_G32 or MXFP4 "
                  "(got %d)",
                  D->expert_w);
    if (D->n_shared && D->shared_w != MOE_BF16 && D->shared_w != MOE_I8_ROW)
      return fail(MOE_EUNSUPPORTED, "act BF16 needs shared weights BF16 or I8_ROW (got %d)",
                  D->shared_w);
    if (D->d % OUT_COLS_BLOCK || D->ffn % H_COLS_BLOCK ||
        (D->n_shared && D->shared_ffn % H_COLS_BLOCK))
      return fail(MOE_EUNSUPPORTED, "BF16 path needs d %% 256 == 0 and ffn, shared_ffn %% 128 == 0");
    const int kstep = kc_of(D->expert_w) * lead_of(D->expert_w, LEAD_I4);
    if (D->ffn % kstep || D->d % kstep) {
      if (D->expert_w == MOE_MXFP4)
        return fail(MOE_EUNSUPPORTED, "MXFP4 routed experts need d, ffn %% %d == 0", kstep);
      return fail(MOE_EUNSUPPORTED, "%d-bit routed experts need ffn %% %d == 0",
                  ig32_bits(D->expert_w), kstep);
    }
  } else {
    return fail(MOE_EUNSUPPORTED, "act dtype %d unsupported", D->act);
  }
  return MOE_OK;
}

moe_status check_tk(const moe_desc* D, int32_t T, int32_t k) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d is negative", T);
  if (k < 1 || k > std::min(D->n_experts, MAX_TOPK))
    return fail(MOE_EINVAL, "k=%d outside [1, min(n_experts, %d)]", k, MAX_TOPK);
  if ((int64_t)T * k > (int64_t)1 << 30)
    return fail(MOE_EINVAL, "T*k=%lld exceeds 2^30", (long long)T * k);
  // activation matrices (hidden, h) are addressed with 32-bit byte offsets
  const int64_t wmax = std::max<int64_t>(D->ffn, D->n_shared ? D->shared_ffn : 0);
  if ((int64_t)T * k * wmax >= (int64_t)1 << 31 || (int64_t)T * D->d >= (int64_t)1 << 31)
    return fail(MOE_EINVAL, "T=%d, k=%d: T*k*ffn and T*d must stay below 2^31 elements", T, k);
  return MOE_OK;
}

moe_status check_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(MOE_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(MOE_EINVAL, "%s is not %zu-byte aligned", name, align);
  return MOE_OK;
}

#define TRY(x)                      \
  do {                              \
    moe_status _s = (x);            \
    if (_s != MOE_OK) return _s;    \
  } while (0)

// int4 / b-bit layers get the fp16 copy of x (and its per-token scales) from
// the route plan's launches.
bool x16_layer(const moe_desc* D) { return D->act == MOE_BF16 && ig32_bits(D->expert_w) != 0; }

moe_status device_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- blob packing --------------------------------------------------------
struct MatIO {
  int fmt;
  int64_t rows, K;
  const uint8_t* q;  // canonical codes / values
  const uint8_t* s;  // canonical scales (I4: [rows, K/32], I8: [rows])
};

// canonical element (row, k): code (I4/I8) or raw bits (BF16) / float (F32)
inline int i4_code(const MatIO& m, int64_t r, int64_t k) {
  uint8_t b = m.q[r * (m.K / 2) + k / 2];
  int n = (k & 1) ? (b >> 4) : (b & 15);
  return n >= 8 ? n - 16 : n;
}
// nibble of a packed lane dword that holds element i (0..7) of the lane's 8
inline int i4_nibble(int i) { return (i & 1) ? 4 + (i >> 1) : (i >> 1); }
// b-bit group-32 tiles: byte offset of dword dw of lane `lane`'s code stream
// (16-byte groups of all lanes, an odd b's last two dwords in 8-byte ones)
inline size_t ig32_dword_offset(int b, int lane, int dw) {
  const int G = (2 * b) / 4;
  return dw < 4 * G ? (size_t)(dw >> 2) * 1024 + lane * 16 + (dw & 3) * 4
                    : (size_t)G * 1024 + lane * 8 + (dw - 4 * G) * 4;
}
inline uint16_t i4_scale(const MatIO& m, int64_t r, int64_t k) {
  return ((const uint16_t*)m.s)[r * (m.K / 32) + k / 32];
}

// Outcome of packing one tile or expert.
enum PackResult { PK_OK = 0, PK_CODE = 1, PK_SCALE = 2 };

// An fp16 scale the kernels can use: finite, and for group-32 codes with
// largest magnitude qmax (0 for per-row int8 scales), |s| * qmax must stay
// below 65520 so that fp16(code * s) -- the gate/up products run on fp16
// weights -- never rounds to infinity.
inline bool f16_scale_ok(uint16_t bits, int qmax) {
  if ((bits & 0x7c00u) == 0x7c00u) return false;  // inf or NaN
  const int e = (bits >> 10) & 31, m = bits & 1023;
  const double mag = e ? ldexp(1024 + m, e - 25) : ldexp(m, -24);
  return mag * qmax < 65520.0;
}

// One 64-row x 64-K wave tile, laid out for the 16x16x32 MFMA.  Fragment f
// (0..3) takes 16 rows from matrix m[f], rows row_of(f, c) for c = 0..15;
// K step s (0..1) covers 32 K.  Lane l of the consuming wave holds row
// c = l % 16 and K offsets 32*s + 8*(l/16) .. +7.
//   BF16: 16-byte piece (f*2 + s, lane) at ((f*2 + s)*64 + lane)*16
//   I4  : dword (code + 8 per nibble; element 2j in nibble j, 2j+1 in j+4) at
//         ((f/2)*64 + lane)*16 + ((f%2)*2 + s)*4; then per row c the 8 fp16
//         group scales [f][s] at 2048 + c*16
//   I8  : 8 int8 codes at (f*64 + lane)*16 + s*8
struct OutIO {  // canonical outputs of unpacking
  uint8_t* q;
  uint8_t* s;
};

// Position in lane l's 2b dwords of bit `k` of u = code + 2^(b-1), the
// offset binary of element i (0..7) of fragment fi = 2 f + s.  Elements 2j
// and 2j+1 form pair P = 4 fi + j; the even element sits in a dword's low
// half-word, the odd one at the same bits of its high half-word, so the
// kernels cut a pair out with one AND-OR.  Each half-word holds NF = 16 / b
// fields of b bits: pair P < 2 b NF at bit b (P % NF) of dword P / NF; the
// remaining pairs take the half-words' SB = 16 - NF b spare top bits in turn,
// bit k of the q-th such pair at spare bit g = q b + k, i.e. bit NF b + g % SB
// of dword g / SB.  (b = 2: dword fi / 2 at 8 (fi % 2) + 2 j; b = 3: five
// fields a half, pairs 30-31 in the spare bits.)
inline int ig32_bit_pos(int b, int fi, int i, int k) {
  const int nf = 16 / b, sb = 16 - nf * b, npf = 2 * b * nf;
  const int P = 4 * fi + (i >> 1), half = 16 * (i & 1);
  if (P < npf) return 32 * (P / nf) + half + b * (P % nf) + k;
  const int g = (P - npf) * b + k;
  return 32 * (g / sb) + half + nf * b + g % sb;
}

// b-bit group-32 tile: lane l's codes of fragment f, K step s, at the bit
// positions of ig32_bit_pos, then the fp16 group scales [row c][f][s] at
// 512 b + c*16.
template <typename RowOf>
int pack_tile_ig32(const MatIO* const m[4], RowOf row_of, int64_t kc, uint8_t* dst) {
  const int b = ig32_bits(m[0]->fmt), lim = (1 << (b - 1)) - 1;
  for (int lane = 0; lane < 64; lane++) {
    uint32_t w[16] = {0};
    for (int f = 0; f < 4; f++) {
      const MatIO& M = *m[f];
      const int64_t r = row_of(f, lane & 15);
      for (int s = 0; s < 2; s++) {
        const int64_t k0 = kc * KC + s * 32 + 8 * (lane >> 4);
        for (int i = 0; i < 8; i++) {
          const int c = ((const int8_t*)M.q)[r * M.K + k0 + i];
          if (c < -lim || c > lim) return PK_CODE;
          const uint32_t u = (uint32_t)(c + (1 << (b - 1)));
          for (int k = 0; k < b; k++) {
            const int pos = ig32_bit_pos(b, 2 * f + s, i, k);
            w[pos >> 5] |= ((u >> k) & 1u) << (pos & 31);
          }
        }
      }
    }
    for (int dw = 0; dw < 2 * b; dw++) memcpy(dst + ig32_dword_offset(b, lane, dw), &w[dw], 4);
  }
  for (int c = 0; c < 16; c++) {
    uint16_t* o = (uint16_t*)(dst + 512 * b + c * 16);
    for (int f = 0; f < 4; f++)
      for (int s = 0; s < 2; s++) {
        o[f * 2 + s] = i4_scale(*m[f], row_of(f, c), kc * KC + s * 32);
        if (!f16_scale_ok(o[f * 2 + s], lim)) return PK_SCALE;
      }
  }
  return PK_OK;
}

// MXFP4 tile (64 rows x 128 K, for the scaled FP4 MFMA 16x16x128): lane l of
// the consuming wave takes row c = l % 16 of each fragment and the 32-K block
// kb = l / 16 of the chunk.  Fragment f's 16 code bytes of lane l (the
// canonical bytes of that row and block, element 2j in the low nibble) at
// f*1024 + l*16; lane l's four E8M0 scales (byte f = fragment f) at
// 4096 + l*4.  Returns false on a NaN (255) scale.
template <typename RowOf>
int pack_tile_mx(const MatIO* const m[4], RowOf row_of, int64_t kc, uint8_t* dst) {
  for (int lane = 0; lane < 64; lane++) {
    const int kb = lane >> 4;
    for (int f = 0; f < 4; f++) {
      const MatIO& M = *m[f];
      const int64_t r = row_of(f, lane & 15);
      memcpy(dst + f * 1024 + lane * 16, M.q + r * (M.K / 2) + kc * (KC_MX / 2) + kb * 16, 16);
      const uint8_t sc = M.s[r * (M.K / 32) + kc * 4 + kb];
      if (sc == 255) return PK_SCALE;
      dst[4096 + lane * 4 + f] = sc;
    }
  }
  return PK_OK;
}

template <typename RowOf>
int pack_tile(const MatIO* const m[4], RowOf row_of, int64_t kc, uint8_t* dst) {
  const int fmt = m[0]->fmt;
  if (fmt == MOE_MXFP4) return pack_tile_mx(m, row_of, kc, dst);
  if (fmt != MOE_I4_G32 && ig32_bits(fmt) != 0) return pack_tile_ig32(m, row_of, kc, dst);
  for (int f = 0; f < 4; f++) {
    const MatIO& M = *m[f];
    for (int lane = 0; lane < 64; lane++) {
      const int64_t r = row_of(f, lane & 15);
      for (int s = 0; s < 2; s++) {
        const int64_t k0 = kc * KC + s * 32 + 8 * (lane >> 4);
        if (fmt == MOE_BF16) {
          memcpy(dst + ((size_t)(f * 2 + s) * 64 + lane) * 16, (const uint16_t*)M.q + r * M.K + k0, 16);
        } else if (fmt == MOE_I4_G32) {
          uint32_t word = 0;  // element 2j in nibble j, element 2j+1 in nibble j+4
          for (int i = 0; i < 8; i++) {
            const int c = i4_code(M, r, k0 + i);
            if (c < -7) return PK_CODE;
            word |= (uint32_t)(c + 8) << (4 * i4_nibble(i));
          }
          memcpy(dst + ((size_t)(f >> 1) * 64 + lane) * 16 + ((f & 1) * 2 + s) * 4, &word, 4);
        } else {  // I8: the codes as they are
          memcpy(dst + ((size_t)f * 64 + lane) * 16 + s * 8, (const int8_t*)M.q + r * M.K + k0, 8);
        }
      }
    }
  }
  if (fmt == MOE_I4_G32) {
    for (int c = 0; c < 16; c++) {
      uint16_t* o = (uint16_t*)(dst + 2048 + c * 16);
      for (int f = 0; f < 4; f++)
        for (int s = 0; s < 2; s++) {
          o[f * 2 + s] = i4_scale(*m[f], row_of(f, c), kc * KC + s * 32);
          if (!f16_scale_ok(o[f * 2 + s], 7)) return PK_SCALE;
        }
    }
  }
  return PK_OK;
}

template <typename RowOf>
void unpack_tile_ig32(const MatIO* const m[4], const OutIO out[4], RowOf row_of, int64_t kc,
                      const uint8_t* src) {
  const int b = ig32_bits(m[0]->fmt);
  for (int lane = 0; lane < 64; lane++) {
    uint32_t w[16] = {0};
    for (int dw = 0; dw < 2 * b; dw++) memcpy(&w[dw], src + ig32_dword_offset(b, lane, dw), 4);
    for (int f = 0; f < 4; f++) {
      const int64_t r = row_of(f, lane & 15), K = m[f]->K;
      for (int s = 0; s < 2; s++) {
        const int64_t k0 = kc * KC + s * 32 + 8 * (lane >> 4);
        for (int i = 0; i < 8; i++) {
          int u = 0;
          for (int k = 0; k < b; k++) {
            const int pos = ig32_bit_pos(b, 2 * f + s, i, k);
            u |= (int)((w[pos >> 5] >> (pos & 31)) & 1u) << k;
          }
          ((int8_t*)out[f].q)[r * K + k0 + i] = (int8_t)(u - (1 << (b - 1)));
        }
      }
    }
  }
  for (int c = 0; c < 16; c++) {
    const uint16_t* o = (const uint16_t*)(src + 512 * b + c * 16);
    for (int f = 0; f < 4; f++)
      for (int s = 0; s < 2; s++)
        ((uint16_t*)out[f].s)[row_of(f, c) * (m[f]->K / 32) + 2 * kc + s] = o[f * 2 + s];
  }
}

template <typename RowOf>
void unpack_tile_mx(const MatIO* const m[4], const OutIO out[4], RowOf row_of, int64_t kc,
                    const uint8_t* src) {
  for (int lane = 0; lane < 64; lane++) {
    const int kb = lane >> 4;
    for (int f = 0; f < 4; f++) {
      const int64_t r = row_of(f, lane & 15), K = m[f]->K;
      memcpy(out[f].q + r * (K / 2) + kc * (KC_MX / 2) + kb * 16, src + f * 1024 + lane * 16, 16);
      out[f].s[r * (K / 32) + kc * 4 + kb] = src[4096 + lane * 4 + f];
    }
  }
}

template <typename RowOf>
void unpack_tile(const MatIO* const m[4], const OutIO out[4], RowOf row_of, int64_t kc,
                 const uint8_t* src) {
  const int fmt = m[0]->fmt;
  if (fmt == MOE_MXFP4) return unpack_tile_mx(m, out, row_of, kc, src);
  if (fmt != MOE_I4_G32 && ig32_bits(fmt) != 0) return unpack_tile_ig32(m, out, row_of, kc, src);
  for (int f = 0; f < 4; f++) {
    const int64_t K = m[f]->K;
    for (int lane = 0; lane < 64; lane++) {
      const int64_t r = row_of(f, lane & 15);
      for (int s = 0; s < 2; s++) {
        const int64_t k0 = kc * KC + s * 32 + 8 * (lane >> 4);
        if (fmt == MOE_BF16) {
          memcpy((uint16_t*)out[f].q + r * K + k0, src + ((size_t)(f * 2 + s) * 64 + lane) * 16, 16);
        } else if (fmt == MOE_I4_G32) {
          uint32_t word;
          memcpy(&word, src + ((size_t)(f >> 1) * 64 + lane) * 16 + ((f & 1) * 2 + s) * 4, 4);
          for (int i = 0; i < 8; i++) {
            const int c = (int)((word >> (4 * i4_nibble(i))) & 15) - 8;
            const int64_t k = k0 + i;
            uint8_t& b = out[f].q[r * (K / 2) + k / 2];
            const uint8_t nib = (uint8_t)(c & 15);
            b = (k & 1) ? (uint8_t)((b & 0x0f) | (nib << 4)) : (uint8_t)((b & 0xf0) | nib);
          }
        } else {
          memcpy((int8_t*)out[f].q + r * K + k0, src + ((size_t)f * 64 + lane) * 16 + s * 8, 8);
        }
      }
    }
  }
  if (fmt == MOE_I4_G32) {
    for (int c = 0; c < 16; c++) {
      const uint16_t* o = (const uint16_t*)(src + 2048 + c * 16);
      for (int f = 0; f < 4; f++)
        for (int s = 0; s < 2; s++)
          ((uint16_t*)out[f].s)[row_of(f, c) * (m[f]->K / 32) + 2 * kc + s] = o[f * 2 + s];
    }
  }
}

size_t canon_q_bytes(int fmt, int64_t rows, int64_t K) {
  switch (fmt) {
    case MOE_F32: return rows * K * 4;
    case MOE_BF16: return rows * K * 2;
    case MOE_I4_G32: return rows * K / 2;
    case MOE_MXFP4: return rows * K / 2;
    default: return rows * K;
  }
}
size_t canon_s_bytes(int fmt, int64_t rows, int64_t K) {
  return ig32_bits(fmt) ? rows * (K / 32) * 2
       : fmt == MOE_I8_ROW ? rows * 2
       : fmt == MOE_MXFP4 ? rows * (K / 32) : 0;
}

struct ExpertIO {  // canonical pointers of one expert (gate, up, down)
  const uint8_t *g, *gs, *u, *us, *dn, *ds;
};

// Pack (or, with unpack = true, unpack) one expert.  Returns PK_CODE on a code
// outside its format's symmetric range, PK_SCALE on a scale the kernels cannot
// use (f16_scale_ok; an MXFP4 scale byte of 255).
int pack_expert(int fmt, int64_t d, int64_t F, ExpertIO io, uint8_t* blob, bool unpack) {
  const size_t w1b = w1_bytes(fmt, d, F);
  if (fmt == MOE_F32) {
    if (!unpack) {
      memcpy(blob, io.g, F * d * 4);
      memcpy(blob + F * d * 4, io.u, F * d * 4);
      memcpy(blob + w1b, io.dn, d * F * 4);
    } else {
      memcpy((void*)io.g, blob, F * d * 4);
      memcpy((void*)io.u, blob + F * d * 4, F * d * 4);
      memcpy((void*)io.dn, blob + w1b, d * F * 4);
    }
    return PK_OK;
  }
  const size_t tb = tile_bytes(fmt);
  const int64_t nk1 = d / kc_of(fmt), nk2 = F / kc_of(fmt);
  const MatIO G{fmt, F, d, io.g, io.gs}, U{fmt, F, d, io.u, io.us}, Dn{fmt, d, F, io.dn, io.ds};
  // W1 run j (h columns c0 = 32*j): fragments 0, 1 = gate rows c0 + 16*(f%2) + c,
  // fragments 2, 3 = up rows of the same columns; runs in order, then K chunks
  const MatIO* const m1[4] = {&G, &G, &U, &U};
  const OutIO og{(uint8_t*)io.g, (uint8_t*)io.gs}, ou{(uint8_t*)io.u, (uint8_t*)io.us};
  const OutIO o1[4] = {og, og, ou, ou};
  for (int64_t j = 0; j < F / H_COLS_WAVE; j++) {
    const int64_t c0 = j * H_COLS_WAVE;
    auto row_of = [c0](int f, int c) { return c0 + (f & 1) * 16 + c; };
    for (int64_t kc = 0; kc < nk1; kc++) {
      uint8_t* t = blob + ((size_t)j * nk1 + kc) * tb;
      if (!unpack) {
        if (const int r = pack_tile(m1, row_of, kc, t)) return r;
      } else {
        unpack_tile(m1, o1, row_of, kc, t);
      }
    }
  }
  // W2 run j: fragment f = down rows 64*j + 16*f + c
  uint8_t* w2 = blob + w1b;
  const MatIO* const m2[4] = {&Dn, &Dn, &Dn, &Dn};
  const OutIO od{(uint8_t*)io.dn, (uint8_t*)io.ds};
  const OutIO o2[4] = {od, od, od, od};
  for (int64_t j = 0; j < d / OUT_COLS_WAVE; j++) {
    const int64_t rbase = j * OUT_COLS_WAVE;
    auto row_of = [rbase](int f, int c) { return rbase + f * 16 + c; };
    for (int64_t kc = 0; kc < nk2; kc++) {
      uint8_t* t = w2 + ((size_t)j * nk2 + kc) * tb;
      if (!unpack) {
        if (const int r = pack_tile(m2, row_of, kc, t)) return r;
      } else {
        unpack_tile(m2, o2, row_of, kc, t);
      }
    }
  }
  if (fmt == MOE_I8_ROW) {  // row scales after the tiles of each section
    uint8_t* s1 = blob + (2 * F / 64) * nk1 * tb;
    uint8_t* s2 = w2 + (d / 64) * nk2 * tb;
    if (!unpack) {
      memcpy(s1, io.gs, F * 2);
      memcpy(s1 + F * 2, io.us, F * 2);
      memcpy(s2, io.ds, d * 2);
      const uint16_t* rs[3] = {(const uint16_t*)io.gs, (const uint16_t*)io.us,
                               (const uint16_t*)io.ds};
      const int64_t nrs[3] = {F, F, d};
      for (int j = 0; j < 3; j++)
        for (int64_t r = 0; r < nrs[j]; r++)
          if (!f16_scale_ok(rs[j][r], 0)) return PK_SCALE;
    } else {
      memcpy((void*)io.gs, s1, F * 2);
      memcpy((void*)io.us, s1 + F * 2, F * 2);
      memcpy((void*)io.ds, s2, d * 2);
    }
  }
  return PK_OK;
}

moe_status pack_or_unpack(const moe_desc* D, int32_t kind, const void* gate, const void* gs,
                          const void* up, const void* us, const void* down, const void* ds,
                          void* blob, size_t blob_bytes, bool unpack) {
  TRY(check_desc(D));
  if (kind != MOE_BLOB_ROUTED && kind != MOE_BLOB_SHARED)
    return fail(MOE_EINVAL, "blob kind %d unknown", kind);
  if (kind == MOE_BLOB_SHARED && !D->n_shared)
    return fail(MOE_EINVAL, "desc has no shared expert");
  const int fmt = kind == MOE_BLOB_ROUTED ? D->expert_w : D->shared_w;
  const int64_t n = kind == MOE_BLOB_ROUTED ? D->n_experts : 1;
  const int64_t d = D->d, F = kind == MOE_BLOB_ROUTED ? D->ffn : D->shared_ffn;
  const size_t need = n * expert_bytes(fmt, d, F);
  if (!blob || !gate || !up || !down) return fail(MOE_EINVAL, "NULL weight or blob pointer");
  if ((ig32_bits(fmt) || fmt == MOE_I8_ROW || fmt == MOE_MXFP4) && (!gs || !us || !ds))
    return fail(MOE_EINVAL, "quantized weights need their scales");
  if (blob_bytes < need) return fail(MOE_EINVAL, "blob_bytes %zu < %zu", blob_bytes, need);
  const size_t gq = canon_q_bytes(fmt, F, d), gsb = canon_s_bytes(fmt, F, d);
  const size_t dq = canon_q_bytes(fmt, d, F), dsb = canon_s_bytes(fmt, d, F);
  const size_t eb = expert_bytes(fmt, d, F);
  std::vector<char> bad(n, 0);
  auto work = [&](int64_t e0, int64_t e1) {
    for (int64_t e = e0; e < e1; e++) {
      ExpertIO io{(const uint8_t*)gate + e * gq, gs ? (const uint8_t*)gs + e * gsb : nullptr,
                  (const uint8_t*)up + e * gq,   us ? (const uint8_t*)us + e * gsb : nullptr,
                  (const uint8_t*)down + e * dq, ds ? (const uint8_t*)ds + e * dsb : nullptr};
      bad[e] = (char)pack_expert(fmt, d, F, io, (uint8_t*)blob + e * eb, unpack);
    }
  };
  const int nt = (int)std::max<int64_t>(1, std::min<int64_t>(n, std::max(1u, std::thread::hardware_concurrency())));
  std::vector<std::thread> th;
  for (int i = 0; i < nt; i++) th.emplace_back(work, n * i / nt, n * (i + 1) / nt);
  for (auto& t : th) t.join();
  for (int64_t e = 0; e < n; e++)
    if (bad[e]) {
      if (fmt == MOE_MXFP4)
        return fail(MOE_EINVAL, "expert %lld holds an MXFP4 scale byte of 255 (NaN)",
                    (long long)e);
      const int b = fmt == MOE_I8_ROW ? 8 : ig32_bits(fmt);
      const int qmax = (1 << (b - 1)) - 1;
      if (bad[e] == PK_SCALE) {
        if (fmt == MOE_I8_ROW)
          return fail(MOE_EINVAL, "expert %lld holds a row scale that is not finite",
                      (long long)e);
        return fail(MOE_EINVAL,
                    "expert %lld holds a group scale that is not finite or whose %d-fold "
                    "overflows fp16 (|scale| * %d must stay below 65520)",
                    (long long)e, qmax, qmax);
      }
      return fail(MOE_EINVAL, "expert %lld holds a code outside [%d, %d]", (long long)e, -qmax,
                  qmax);
    }
  return ok();
}

}  // namespace

moe_status moe::grouped_ffn_call(const moe_desc* D, int32_t T, int32_t k, const void* hidden,
                                 const float* topk_w, const int32_t* offsets, const int32_t* perm,
                                 const void* routed_blob, const void* shared_blob,
                                 float* out_assign, float* shared_out, void* workspace,
                                 size_t ws_bytes, ScratchFn scratch, void* stream) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  TRY(check_ptr(hidden, "hidden"));
  TRY(check_ptr(topk_w, "topk_w"));
  TRY(check_ptr(offsets, "offsets"));
  TRY(check_ptr(perm, "perm"));
  TRY(check_ptr(routed_blob, "routed_blob"));
  TRY(check_ptr(out_assign, "out_assign"));
  if (!scratch) TRY(check_ptr(workspace, "workspace", 256));
  if (D->n_shared) {
    TRY(check_ptr(shared_blob, "shared_blob"));
    TRY(check_ptr(shared_out, "shared_out"));
  } else if (shared_blob || shared_out) {
    return fail(MOE_EINVAL, "shared_blob/shared_out must be NULL when n_shared == 0");
  }
  const WsLayout L = ws_layout(*D, T, k);
  if (ws_bytes < L.total) {
    if (scratch)
      return fail(MOE_EWORKSPACE,
                  "T=%d, k=%d need %zu bytes of scratch; the library's static scratch holds "
                  "%zu (use moe_grouped_ffn with a workspace)",
                  T, k, L.total, ws_bytes);
    return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  }
  if (T == 0) return ok();
  if (scratch) {
    const hipError_t e = scratch(&workspace);
    if (e != hipSuccess) return device_result(e, "scratch address");
  }
  uint8_t* w = (uint8_t*)workspace;
  FfnArgs a{};
  a.T = T; a.k = k; a.d = D->d; a.E = D->n_experts; a.F = D->ffn;
  a.Fs = D->n_shared ? D->shared_ffn : 0; a.n_shared = D->n_shared;
  a.routed_fmt = D->expert_w; a.shared_fmt = D->shared_w;
  a.routed_slots = L.routed_slots;
  a.shared_slots = D->n_shared ? (T + BM - 1) / BM : 0;
  a.hidden = hidden; a.topk_w = topk_w; a.offsets = offsets; a.perm = perm;
  a.tiles = (const int4*)(w + L.tiles);
  a.routed_blob = (const uint8_t*)routed_blob;
  a.shared_blob = (const uint8_t*)shared_blob;
  a.h_routed = w + L.h_routed; a.h_shared = w + L.h_shared;
  a.x16 = (uint16_t*)(w + L.x16); a.xscale = (float*)(w + L.xexp);
  a.xq = w + L.x16; a.xsc = w + L.xexp;
  a.hq = w + L.h_routed; a.hsc = w + L.h_scale;
  a.out_assign = out_assign; a.shared_out = shared_out;
  hipStream_t s = (hipStream_t)stream;
  if (scratch) {
    const hipError_t e = launch_tiles_from_offsets(
        D->n_experts, tile_rows(T), L.routed_slots, offsets, (int4*)(w + L.tiles), T, D->d,
        x16_layer(D) ? (const uint16_t*)hidden : nullptr, a.x16, a.xscale, s);
    if (e != hipSuccess) return device_result(e, "row-tile plan launch");
  }
  return device_result(D->act == MOE_F32 ? launch_ffn_f32(a, s) : launch_ffn_bf16(a, s),
                       "grouped-ffn launch");
}

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EDEVICE: return "device error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_blob_bytes(const moe_desc* D, int32_t kind, size_t* bytes) {
  TRY(check_desc(D));
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  if (kind == MOE_BLOB_ROUTED) {
    *bytes = (size_t)D->n_experts * expert_bytes(D->expert_w, D->d, D->ffn);
  } else if (kind == MOE_BLOB_SHARED) {
    *bytes = D->n_shared ? expert_bytes(D->shared_w, D->d, D->shared_ffn) : 0;
  } else {
    return fail(MOE_EINVAL, "blob kind %d unknown", kind);
  }
  return ok();
}

moe_status moe_pack_experts(const moe_desc* D, int32_t kind, const void* gate, const void* gs,
                            const void* up, const void* us, const void* down, const void* ds,
                            void* blob, size_t blob_bytes) {
  return pack_or_unpack(D, kind, gate, gs, up, us, down, ds, blob, blob_bytes, false);
}

moe_status moe_unpack_experts(const moe_desc* D, int32_t kind, const void* blob, size_t blob_bytes,
                              void* gate, void* gs, void* up, void* us, void* down, void* ds) {
  return pack_or_unpack(D, kind, gate, gs, up, us, down, ds, (void*)blob, blob_bytes, true);
}

moe_status moe_workspace_bytes(const moe_desc* D, int32_t T, int32_t k, size_t* bytes) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = ws_layout(*D, T, k).total;
  return ok();
}

moe_status moe_route(const moe_desc* D, int32_t T, int32_t k, const void* hidden,
                     const void* router_w, const float* bias, float* logits, int32_t* topk_ids,
                     float* topk_w, void* stream) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  TRY(check_ptr(hidden, "hidden"));
  TRY(check_ptr(router_w, "router_w"));
  if (bias) TRY(check_ptr(bias, "bias", 4));
  TRY(check_ptr(logits, "logits"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_w, "topk_w"));
  if (T == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = D->act == MOE_F32
                     ? launch_router_f32(T, D->d, D->n_experts, (const float*)hidden,
                                         (const float*)router_w, bias, logits, s)
                     : launch_router_bf16(T, D->d, D->n_experts, hidden, router_w, bias, logits, s);
  if (e != hipSuccess) return device_result(e, "router launch");
  return device_result(launch_topk(T, D->n_experts, k, logits, topk_ids, topk_w, s),
                       "top-k launch");
}

moe_status moe_route_from_logits(const moe_desc* D, int32_t T, int32_t k, const float* logits,
                                 int32_t* topk_ids, float* topk_w, void* stream) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  TRY(check_ptr(logits, "logits"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_w, "topk_w"));
  if (T == 0) return ok();
  return device_result(
      launch_topk(T, D->n_experts, k, logits, topk_ids, topk_w, (hipStream_t)stream),
      "top-k launch");
}

moe_status moe_permute(const moe_desc* D, int32_t T, int32_t k, const void* hidden,
                       const int32_t* topk_ids, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, void* workspace, size_t ws_bytes, void* stream) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  TRY(check_ptr(hidden, "hidden"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(offsets, "offsets"));
  TRY(check_ptr(perm, "perm"));
  TRY(check_ptr(inv_perm, "inv_perm"));
  TRY(check_ptr(workspace, "workspace", 256));
  const WsLayout L = ws_layout(*D, T, k);
  if (ws_bytes < L.total)
    return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if (T == 0) return ok();
  const uint16_t* xs = x16_layer(D) ? (const uint16_t*)hidden : nullptr;
  return device_result(launch_plan(T, k, D->n_experts, tile_rows(T), topk_ids, offsets, perm,
                                   inv_perm, workspace, L, D->d, xs, (hipStream_t)stream),
                       "route-plan launch");
}

moe_status moe_route_plan(const moe_desc* D, int32_t T, int32_t k, const void* hidden,
                          const void* router_w, const float* bias, float* logits,
                          int32_t* topk_ids, float* topk_w, int32_t* offsets, int32_t* perm,
                          int32_t* inv_perm, void* workspace, size_t ws_bytes, void* stream) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  TRY(check_ptr(hidden, "hidden"));
  TRY(check_ptr(router_w, "router_w"));
  if (bias) TRY(check_ptr(bias, "bias", 4));
  TRY(check_ptr(logits, "logits"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_w, "topk_w"));
  TRY(check_ptr(offsets, "offsets"));
  TRY(check_ptr(perm, "perm"));
  TRY(check_ptr(inv_perm, "inv_perm"));
  TRY(check_ptr(workspace, "workspace", 256));
  const WsLayout L = ws_layout(*D, T, k);
  if (ws_bytes < L.total)
    return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if (T == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  if (D->act == MOE_BF16 && T <= 32)
    return device_result(
        launch_route_plan_small(T, D->d, D->n_experts, k, hidden, router_w, bias, logits,
                                topk_ids, topk_w, offsets, perm, inv_perm, tile_rows(T),
                                workspace, L, x16_layer(D), s),
        "route-plan launch");
  TRY(moe_route(D, T, k, hidden, router_w, bias, logits, topk_ids, topk_w, stream));
  return moe_permute(D, T, k, hidden, topk_ids, offsets, perm, inv_perm, workspace, ws_bytes,
                     stream);
}

moe_status moe_grouped_ffn(const moe_desc* D, int32_t T, int32_t k, const void* hidden,
                           const float* topk_w, const int32_t* offsets, const int32_t* perm,
                           const void* routed_blob, const void* shared_blob, float* out_assign,
                           float* shared_out, void* workspace, size_t ws_bytes, void* stream) {
  return grouped_ffn_call(D, T, k, hidden, topk_w, offsets, perm, routed_blob, shared_blob,
                          out_assign, shared_out, workspace, ws_bytes, nullptr, stream);
}

moe_status moe_combine(const moe_desc* D, int32_t T, int32_t k, const float* out_assign,
                       const int32_t* inv_perm, const float* shared_out, void* y, void* stream) {
  TRY(check_desc(D));
  TRY(check_tk(D, T, k));
  TRY(check_ptr(out_assign, "out_assign"));
  TRY(check_ptr(inv_perm, "inv_perm"));
  TRY(check_ptr(y, "y"));
  if (D->n_shared) TRY(check_ptr(shared_out, "shared_out"));
  else if (shared_out) return fail(MOE_EINVAL, "shared_out must be NULL when n_shared == 0");
  if (T == 0) return ok();
  return device_result(launch_combine(T, k, D->d, D->act, out_assign, inv_perm, shared_out, y,
                                      (hipStream_t)stream),
                       "combine launch");
}

}  // extern "C"
