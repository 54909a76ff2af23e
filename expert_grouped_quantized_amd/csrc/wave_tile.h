// wave_tile.h -- one wave's share of an expert-grouped GEMM tile: the MFMA
// wrappers, the weight-tile registers with their in-register dequantization,
// and the epilogue that stores a wave's 64 weight rows x (16 * NMF) tile rows.
// Kept apart from the kernels that use it so their row tiles of every size
// share one arithmetic.
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_f __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4_t mfma16x16(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_f, a),
                                                 __builtin_bit_cast(bf16x8_f, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16x16_f16(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Weight loads; NT streams them past the caches (non-temporal) for weights that
// one row tile reads once, so they do not evict activation rows.
template <bool NT>
__device__ __forceinline__ u32x4_t ldw(const uint8_t* base, int i) {
  if (NT) return __builtin_nontemporal_load((const u32x4_t*)base + i);
  return ((const u32x4_t*)base)[i];
}

// A stream of 16-byte loads addressed as a buffer: `rsrc` holds a scalar
// base (a wave's run of weight tiles, or an activation matrix) and `soff` the
// scalar byte offset of the current chunk, so a load takes only the lane's
// 32-bit offset from a vector register -- no 64-bit per-lane address, and the
// chunk advance is scalar arithmetic.  The whole 32-bit offset range is in
// bounds (the ABI keeps every activation matrix below 4 GiB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffff,
                                           0x00020000);
}
struct BufSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t soff;
  // NT: non-temporal (streamed past the caches)
  template <bool NT>
  __device__ __forceinline__ u32x4_t ld16(uint32_t voff) const {
    return __builtin_bit_cast(u32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, NT ? 2 : 0));
  }
  template <bool NT>
  __device__ __forceinline__ uint64_t ld8(uint32_t voff) const {
    return __builtin_bit_cast(uint64_t,
                              __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, NT ? 2 : 0));
  }
};

// Constants of the int4 -> fp16 conversion, kept in registers (VOP3
// encodings take no literal operands): the low- and high-nibble masks of a
// pair and the fp16 exponents of 1024 and 64 in both halves.
struct F16Consts {
  uint32_t lo, hi, magic, magic64;
};

// Group scale si (0..7) of the 8 fp16 scales in sc, in both halves of a
// packed pair: the dword goes through a scalar (hipcc compiles a bit_cast of
// an ext-vector element as a read of element 0), and the half is picked by a
// shuffle that the packed multiply takes as its op_sel, one op fewer than an
// integer splat.
__device__ __forceinline__ f16x2_t scale_splat(const u32x4_t& sc, int si) {
  const uint32_t dw = sc[si >> 1];
  const f16x2_t p = __builtin_bit_cast(f16x2_t, dw);
  return (si & 1) ? __builtin_shufflevector(p, p, 1, 1) : __builtin_shufflevector(p, p, 0, 0);
}

// ---- weight registers of one wave tile (64 rows x 64 K) -------------------
// Fragment f (0..3) is 16 weight rows; step s (0..1) is 32 K.  Lane l holds
// row l % 16 of each fragment and K elements 32*s + 8*(l/16) .. +7.
// frag() returns the 8 weights as bf16 (for bf16 MFMA), frag16() as fp16.
template <int FMT>
struct WTile;

template <>
struct WTile<MOE_BF16> {
  u32x4_t v[8];  // [frag][step]
  template <bool NT>
  __device__ __forceinline__ void load(const BufSrc& t, int lane) {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = t.ld16<NT>((uint32_t)(lane * 16 + j * 1024));
  }
  __device__ __forceinline__ u32x4_t frag(int f, int s, const F16Consts&) const {
    return v[f * 2 + s];
  }
  __device__ __forceinline__ u32x4_t frag16(int f, int s, const F16Consts&) const {
    return v[f * 2 + s];  // never used: bf16 weights run bf16 MFMA
  }
};

template <>
struct WTile<MOE_I4_G32> {
  // [frag pair]; dword (f%2)*2 + s holds the lane's 8 codes + 8: element 2j in
  // nibble j, element 2j+1 in nibble j+4 (so nibbles j and j+4, at bits 4j and
  // 16+4j, are the pair that one packed fp16 register takes)
  u32x4_t v[2];
  u32x4_t sc;  // 8 fp16 group scales, index f*2 + s (group = step)
  template <bool NT>
  __device__ __forceinline__ void load(const BufSrc& t, int lane) {
    v[0] = t.ld16<NT>((uint32_t)(lane * 16));
    v[1] = t.ld16<NT>((uint32_t)(lane * 16 + 1024));
    sc = t.ld16<NT>((uint32_t)((lane & 15) * 16 + 2048));
  }
  __device__ __forceinline__ uint32_t scale_bits(int f, int s) const {
    const int si = f * 2 + s;
    const uint32_t sw = sc[si >> 1];
    return (si & 1) ? (sw >> 16) : (sw & 0xffffu);
  }
  // bf16(code * scale): a nibble pair OR-ed under the fp16 exponent of 1024
  // reads as 1024 + code + 8 each; one mixed-precision FMA per half takes it
  // with the fp16 scale and -1032 * scale (both products exact in fp32, so the
  // sum is code * scale exactly) and the pack rounds to nearest even.  The
  // pairs in the high nibbles of bytes 0 and 2 are taken in place under the
  // exponent of 64, where those bits count 1 to 8: 64 + code + 8, made exact
  // with -72 * scale, so one shift per dword serves all four pairs.  Both
  // biases are mixed-precision FMAs of the fp16 scale (no conversion).
  __device__ __forceinline__ u32x4_t frag(int f, int s, const F16Consts& k) const {
    const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)scale_bits(f, s));
    const float scale = (float)sh;
    const float bias_lo = fmaf((float)sh, -1032.0f, 0.0f);
    const float bias_hi = fmaf((float)sh, -72.0f, 0.0f);
    const uint32_t q = v[f >> 1][(f & 1) * 2 + s];
    const uint32_t q8 = q >> 8;
    const uint32_t w[4] = {and_or_b32(q, k.lo, k.magic), and_or_b32(q, k.hi, k.magic64),
                           and_or_b32(q8, k.lo, k.magic), and_or_b32(q8, k.hi, k.magic64)};
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t wj = w[j];
      const f16x2_t t = __builtin_bit_cast(f16x2_t, wj);
      const float b = (j & 1) ? bias_hi : bias_lo;
      r[j] = pack_bf16x2(fmaf((float)t[0], scale, b), fmaf((float)t[1], scale, b));
    }
    return r;
  }
  // fp16(code * scale): a nibble pair OR-ed into two fp16 mantissas is
  // (1024 + code + 8) each; one packed subtract makes the codes exact, one
  // packed multiply by the fp16 scale rounds each product to nearest even.
  // The pairs held in the high nibbles of bytes 0 and 2 are taken in place,
  // as 1024 + 16 (code + 8), and made exact with one packed fma by 1/16 and
  // -72 instead of a shift: one shift per dword instead of three.
  __device__ __forceinline__ u32x4_t frag16(int f, int s, const F16Consts& k) const {
    const f16x2_t s2 = scale_splat(sc, f * 2 + s);
    const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t q = v[f >> 1][(f & 1) * 2 + s];
    const uint32_t q8 = q >> 8;
    const f16x2_t t0 = __builtin_bit_cast(f16x2_t, and_or_b32(q, k.lo, k.magic));
    const f16x2_t t1 = __builtin_bit_cast(f16x2_t, and_or_b32(q, k.hi, k.magic));
    const f16x2_t t2 = __builtin_bit_cast(f16x2_t, and_or_b32(q8, k.lo, k.magic));
    const f16x2_t t3 = __builtin_bit_cast(f16x2_t, and_or_b32(q8, k.hi, k.magic));
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, (t0 + off) * s2);
    r[1] = __builtin_bit_cast(uint32_t, (t1 * sixteenth + off16) * s2);
    r[2] = __builtin_bit_cast(uint32_t, (t2 + off) * s2);
    r[3] = __builtin_bit_cast(uint32_t, (t3 * sixteenth + off16) * s2);
    return r;
  }
};

template <>
struct WTile<MOE_I8_ROW> {
  u32x4_t v[4];  // [frag]; dwords 2s, 2s+1 hold 8 int8 codes
  template <bool NT>
  __device__ __forceinline__ void load(const BufSrc& t, int lane) {
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = t.ld16<NT>((uint32_t)(lane * 16 + j * 1024));
  }
  __device__ __forceinline__ u32x4_t frag(int f, int s, const F16Consts&) const {
    const uint32_t w0 = v[f][2 * s], w1 = v[f][2 * s + 1];
    u32x4_t r;
    r[0] = pack_bf16x2(sbyte0_f(w0), sbyte1_f(w0));
    r[1] = pack_bf16x2(sbyte2_f(w0), sbyte3_f(w0));
    r[2] = pack_bf16x2(sbyte0_f(w1), sbyte1_f(w1));
    r[3] = pack_bf16x2(sbyte2_f(w1), sbyte3_f(w1));
    return r;
  }
  // fp16(code), exact: flipping a byte's sign bit gives code + 128 in
  // [0, 255]; a byte permute sets it under the fp16 exponent byte 0x64, which
  // reads as 1024 + code + 128, and one packed subtract of 1152 leaves the
  // code.  (All compiler-visible ops: the MFMA that reads the result right
  // after gets its hazard wait states.)
  __device__ __forceinline__ u32x4_t frag16(int f, int s, const F16Consts&) const {
    const uint32_t w0 = v[f][2 * s] ^ 0x80808080u, w1 = v[f][2 * s + 1] ^ 0x80808080u;
    const uint32_t hi = 0x64646464u;
    const f16x2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    // selector bytes 4..7 pick bytes of the first operand, 0..3 of the second
    auto half2 = [&](uint32_t w, uint32_t sel) {
      return __builtin_bit_cast(uint32_t,
                                __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(w, hi, sel)) + off);
    };
    return u32x4_t{half2(w0, 0x00050004u), half2(w0, 0x00070006u), half2(w1, 0x00050004u),
                   half2(w1, 0x00070006u)};
  }
};

// ---- b-bit group-32 codes (b = 2, 3, 5, 6, 7, 8) -------------------------
// Lane l's 64 codes of a wave tile, each as u = code + 2^(b-1) (offset
// binary), fill 2b dwords: the dwords sit in 16-byte groups (group g of all
// lanes at g*1024 + lane*16), an odd b ending with one 8-byte group (at
// G*1024 + lane*8); the fp16 group scales follow at 512 b ([row c][f][s] at
// 512 b + c*16), as in the int4 tile.  So every load is a coalesced wave-wide
// run and the blob holds exactly b bits per weight plus the scales.
// Elements 2j and 2j+1 of fragment fi = 2 f + s form pair P = 4 fi + j of the
// lane's 32; the even element sits in a dword's low half-word and the odd one
// at the same bits of its high half-word, so one AND-OR with a field mask (in
// both halves) and the fp16 exponent of 1024 cuts a pair out as two fp16
// values 1024 + 2^p u, exact (p + b <= 10).  Each half-word holds NF = 16 / b
// fields of b bits: pair P < 2 b NF has u in dword P / NF at bit b (P % NF)
// (a field that ends past bit 10 is read from the dword shifted down to bit
// 0); the last 32 - 2 b NF pairs take the half-words' SB = 16 - NF b spare
// top bits in turn: bit k of the q-th such pair's u is spare bit g = q b + k,
// at bit NF b + g % SB of dword g / SB.  (b = 2: 8 fields a half; b = 3: 5
// fields, pairs 30-31 in the spare bits; b = 8: 2 fields.)  ig32_bit_pos in
// the packer is the same map.
template <int B>
struct WTileP {
  static_assert(B >= 2 && B <= 8 && B != 4, "group-32 codes of 2, 3, 5, 6, 7 or 8 bits");
  static constexpr int NDW = 2 * B;    // dwords per lane
  static constexpr int G = NDW / 4;    // full 16-byte groups
  static constexpr bool TAIL = NDW % 4 != 0;
  static constexpr int NF = 16 / B;    // fields per half-word
  static constexpr int SB = 16 - NF * B;  // spare top bits per half-word
  static constexpr int NPF = 2 * B * NF;  // pairs held in fields
  static_assert(NPF + (NDW * SB) / B == 32 && (NDW * SB) % B == 0, "every pair has its bits");
  uint32_t w[NDW];
  u32x4_t sc;
  template <bool NT>
  __device__ __forceinline__ void load(const BufSrc& t, int lane) {
#pragma unroll
    for (int g = 0; g < G; g++) {
      const u32x4_t v = t.ld16<NT>((uint32_t)(g * 1024 + lane * 16));
#pragma unroll
      for (int c = 0; c < 4; c++) w[4 * g + c] = v[c];
    }
    if constexpr (TAIL) {
      const uint64_t v = t.ld8<NT>((uint32_t)(G * 1024 + lane * 8));
      w[4 * G] = (uint32_t)v;
      w[4 * G + 1] = (uint32_t)(v >> 32);
    }
    sc = t.ld16<NT>((uint32_t)(512 * B + (lane & 15) * 16));
  }
  __device__ __forceinline__ uint32_t scale_bits(int f, int s) const {
    const int si = f * 2 + s;
    const uint32_t sw = sc[si >> 1];
    return (si & 1) ? (sw >> 16) : (sw & 0xffffu);
  }
  // pair j of fragment (f, s) as two fp16 values 1024 + 2^p u under the
  // exponent of 1024 (p: the bit of u in its half, a constant once unrolled)
  __device__ __forceinline__ uint32_t pair_bits(int f, int s, int j, int& p) const {
    constexpr uint32_t magic = 0x64006400u;
    constexpr uint32_t lowb = (1u << B) - 1u;
    const int P = 4 * (2 * f + s) + j;
    if (SB == 0 || P < NPF) {
      const int o = B * (P % NF);
      const uint32_t d = w[P / NF];
      const bool in_place = o + B <= 10;
      p = in_place ? o : 0;
      return and_or_b32(in_place ? d : d >> o, (lowb << p) * 0x00010001u, magic);
    }
    uint32_t t = magic;
    p = 0;
    if constexpr (SB > 0) {
      // gather the spare bits of pair q, one run of bits per dword
      const int q = P - NPF;
#pragma unroll
      for (int k = 0; k < B;) {
        const int g = q * B + k, d = g / SB, off = g % SB;
        const int n = min(B - k, SB - off);  // bits of u in this dword
        const int pos = NF * B + off;         // their first bit in each half
        t = and_or_b32(w[d] >> (pos - k), (((1u << n) - 1u) << k) * 0x00010001u, t);
        k += n;
      }
    }
    return t;
  }
  // fp16(code * scale): (1024 + 2^p u) 2^-p - (1024 2^-p + 2^(b-1)) is the
  // code, exact (one packed fma); one packed multiply by the scale rounds
  // each product to nearest even
  __device__ __forceinline__ u32x4_t frag16(int f, int s, const F16Consts&) const {
    const f16x2_t s2 = scale_splat(sc, f * 2 + s);
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int p;
      const uint32_t t = pair_bits(f, s, j, p);
      const _Float16 k = (_Float16)(1.0f / (float)(1 << p));
      const _Float16 o = (_Float16)(-(1024.0f / (float)(1 << p) + (float)(1 << (B - 1))));
      const f16x2_t c = __builtin_bit_cast(f16x2_t, t) * f16x2_t{k, k} + f16x2_t{o, o};
      r[j] = __builtin_bit_cast(uint32_t, c * s2);
    }
    return r;
  }
  // bf16(code * scale): one mixed-precision fma per value takes the fp16
  // 1024 + 2^p u with scale 2^-p and the bias -(1024 2^-p + 2^(b-1)) scale
  // (every product exact in fp32, so the sum is code * scale exactly); the
  // pack rounds to nearest even
  __device__ __forceinline__ u32x4_t frag(int f, int s, const F16Consts&) const {
    const float scale = f16_bits_to_f32((uint16_t)scale_bits(f, s));
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int p;
      const f16x2_t t = __builtin_bit_cast(f16x2_t, pair_bits(f, s, j, p));
      const float sp = scale * (1.0f / (float)(1 << p));
      const float b = scale * -(1024.0f / (float)(1 << p) + (float)(1 << (B - 1)));
      r[j] = pack_bf16x2(fmaf((float)t[0], sp, b), fmaf((float)t[1], sp, b));
    }
    return r;
  }
};
template <> struct WTile<MOE_I2_G32> : WTileP<2> {};
template <> struct WTile<MOE_I3_G32> : WTileP<3> {};
template <> struct WTile<MOE_I5_G32> : WTileP<5> {};
template <> struct WTile<MOE_I6_G32> : WTileP<6> {};
template <> struct WTile<MOE_I7_G32> : WTileP<7> {};
template <> struct WTile<MOE_I8_G32> : WTileP<8> {};

// Gate/up of int4 (and b-bit group-32) layers runs fp16 MFMA on the fp16
// copy of x: their code -> fp16 conversion costs fewer VALU ops than bf16,
// which sets the speed of the large-T loop and still shows in the
// weight-streaming small-T one.
__host__ __device__ constexpr bool x16_path(int routed_fmt, int) {
  return ig32_bits(routed_fmt) != 0;
}

__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Stores one wave's finished tile.  Accumulator r of fragment (i, f) is tile
// row i*16 + 4*(lane/16) + r and column 16*f + lane%16 of the wave's 64
// weight rows (run `run` of its matrix).
//   stage 1: fragments 0,1 are gate rows and 2,3 the up rows of the same 32
//            h columns; h = w * silu(g) * u in fp32, stored as bf16.  F16
//            tiles ran on activations scaled by 1/xs(i, r): g and u are
//            multiplied back first.  wrow(i, r) is the row's folded weight.
//   stage 2: fp32 output rows.
// int8 tiles apply their per-row fp16 scale here.  Values are stored two
// columns at a time: lanes l and l^1 (columns c, c+1) trade values through
// DPP, the even lane writes rows r = 0, 1 of the pair and the odd lane rows
// 2, 3, each as one store (bf16: 4 bytes, fp32: 8).  Rows at or past `cnt`
// are not stored.
template <int FMT, int STAGE, int NMF, bool F16, typename RowW, typename RowS>
__device__ __forceinline__ void store_wave_tile(const FfnArgs& A, bool shared, int start, int cnt,
                                                int run, int Fw, const uint8_t* sect,
                                                const f32x4_t (&acc)[NMF][4], RowW wrow,
                                                RowS xs) {
  const int lane = threadIdx.x & 63;
  const bool odd = lane & 1;
  auto store_pairs = [&](auto* base, size_t ld, int col, int mrow, const float (&v)[4]) {
    // base: row 0 of this tile; col: this lane's column; mrow: row of v[0]
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int r = odd ? 2 + q : q;  // the row this lane writes
      // each lane sends the value its partner needs: the even lane row 2+q,
      // the odd lane row q (quad_perm [1,0,3,2] swaps neighbours)
      const float va = v[q], vb = v[2 + q];
      const float other = __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, odd ? va : vb), 0xB1, 0xF, 0xF,
                                          false));
      const float mine = odd ? vb : va;
      const float lo = odd ? other : mine, hi = odd ? mine : other;
      auto* dst = base + (size_t)(mrow + r) * ld + (col & ~1);
      if (mrow + r < cnt) {
        if constexpr (sizeof(*base) == 2)
          *(uint32_t*)dst = pack_bf16x2(lo, hi);
        else
          *(float2*)dst = make_float2(lo, hi);
      }
    }
  };
  const size_t tb = tile_bytes(FMT);
  const uint16_t* rscale =
      FMT == MOE_I8_ROW
          ? (const uint16_t*)(sect + (size_t)(STAGE == 1 ? (2 * Fw / 64) * (A.d / KC)
                                                         : (A.d / 64) * (Fw / KC)) * tb)
          : nullptr;
  const int quad = 4 * (lane >> 4);
  if (STAGE == 1) {
    uint16_t* hout = (uint16_t*)(shared ? A.h_shared : A.h_routed);
#pragma unroll
    for (int f = 0; f < 2; f++) {
      const int col = run * H_COLS_WAVE + f * 16 + (lane & 15);
      float sg = 1.0f, su = 1.0f;
      if (FMT == MOE_I8_ROW) {
        sg = f16_bits_to_f32(rscale[col]);
        su = f16_bits_to_f32(rscale[Fw + col]);
      }
#pragma unroll
      for (int i = 0; i < NMF; i++) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          float g = acc[i][f][r] * sg, u = acc[i][f + 2][r] * su;
          if (F16) {
            g *= xs(i, r);
            u *= xs(i, r);
          }
          hv[r] = wrow(i, r) * silu_fast(g) * u;
        }
        store_pairs(hout + (size_t)start * Fw, Fw, col, i * 16 + quad, hv);
      }
    }
  } else {
    float* out = shared ? A.shared_out : A.out_assign;
#pragma unroll
    for (int f = 0; f < 4; f++) {
      const int col = run * OUT_COLS_WAVE + f * 16 + (lane & 15);
      const float sc = FMT == MOE_I8_ROW ? f16_bits_to_f32(rscale[col]) : 1.0f;
#pragma unroll
      for (int i = 0; i < NMF; i++) {
        const float ov[4] = {acc[i][f][0] * sc, acc[i][f][1] * sc, acc[i][f][2] * sc,
                             acc[i][f][3] * sc};
        store_pairs(out + (size_t)start * A.d, A.d, col, i * 16 + quad, ov);
      }
    }
  }
}

}  // namespace moe
