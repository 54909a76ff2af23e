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

// ---- b-bit group-32 codes (b = 5, 6, 7, 8) ------------------------------
// Lane l's codes of a wave tile form one little-endian bit stream of 64 b
// bits: code i (0..7) of fragment f, K step s at bit (2 f + s) 8 b + i b, as
// code + 2^(b-1) (offset binary).  The stream's dwords sit in 16-byte groups
// (group g of all lanes at g*1024 + lane*16), an odd b ending with one
// 8-byte group (at G*1024 + lane*8); the fp16 group scales follow at 512 b,
// as in the int4 tile.  So every load is a coalesced wave-wide run and the
// blob holds exactly b bits per weight plus the scales.
template <int B>
struct WTileB {
  static constexpr int NDW = 2 * B;    // stream dwords per lane
  static constexpr int G = NDW / 4;    // full 16-byte groups
  static constexpr bool TAIL = NDW % 4 != 0;
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
  // bits [o, o + n) of the stream, n <= 16 (o, n constant once unrolled)
  __device__ __forceinline__ uint32_t field(int o, int n) const {
    const int d = o >> 5, sh = o & 31;
    const uint32_t win = sh + n <= 32 ? w[d] >> sh : __builtin_amdgcn_alignbit(w[d + 1], w[d], sh);
    return win & ((1u << n) - 1);
  }
  // fp16(code * scale): each pair of codes under the fp16 exponent of 1024
  // reads as 1024 + code + 2^(b-1); one packed subtract makes the codes exact,
  // one packed multiply by the scale rounds each product to nearest even.
  __device__ __forceinline__ u32x4_t frag16(int f, int s, const F16Consts&) const {
    // integer splat of the scale: the op_sel form (scale_splat) makes the
    // 96-row 2- and 7-bit gate/up kernels spill
    const uint32_t sb = scale_bits(f, s);
    const f16x2_t s2 = __builtin_bit_cast(f16x2_t, sb | (sb << 16));
    constexpr _Float16 bias = (_Float16)(-(1024 + (1 << (B - 1))));
    const f16x2_t off = {bias, bias};
    const int base = (2 * f + s) * 8 * B;
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t lo = field(base + 2 * j * B, B), hi = field(base + (2 * j + 1) * B, B);
      const uint32_t t = ((hi << 16) | lo) | 0x64006400u;
      r[j] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, t) + off) * s2);
    }
    return r;
  }
  // bf16(code * scale): code + 2^(b-1) as a float, one FMA with the scale
  // (exact in fp32), rounded to nearest even by the pack
  __device__ __forceinline__ u32x4_t frag(int f, int s, const F16Consts&) const {
    const float scale = f16_bits_to_f32((uint16_t)scale_bits(f, s));
    const float bias = -(float)(1 << (B - 1)) * scale;
    const int base = (2 * f + s) * 8 * B;
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float a = (float)field(base + 2 * j * B, B), b = (float)field(base + (2 * j + 1) * B, B);
      r[j] = pack_bf16x2(fmaf(a, scale, bias), fmaf(b, scale, bias));
    }
    return r;
  }
};
// ---- 2- and 3-bit codes: laid out for pair extraction ---------------------
// Elements 2j and 2j+1 of a fragment (pair j) sit at the same bits of a
// dword's low and high halves, so one AND-OR with a field mask (in both
// halves) and the fp16 exponent of 1024 gives the pair as two fp16 values
// 1024 + 2^p u, exact, for u = code + 2^(b-1) at bit p <= 7 of its half.
//   b = 2: u of pair j of fragment fi = 2 f + s in stream dword fi / 2 at
//   bit 8 (fi % 2) + 2 j of each half.
//   b = 3: pair P = 4 fi + j of the lane's 32; pairs 0-29 fill five 3-bit
//   fields a half (u at bit 3 (P % 5) of dword P / 5; the fields at bits 9
//   and 12 are read from the dword shifted right by 9), pairs 30 and 31 the
//   halves' spare top bits: bit k of u at bit 15 of dword 3 (P - 30) + k.
// Group scales as in WTileB: [row c][f][s] at 512 b + c*16.
template <int B>
struct WTileP {
  static_assert(B == 2 || B == 3, "pair-extraction tiles hold 2- or 3-bit codes");
  static constexpr int NDW = 2 * B;
  uint32_t w[NDW];
  u32x4_t sc;
  template <bool NT>
  __device__ __forceinline__ void load(const BufSrc& t, int lane) {
    const u32x4_t v = t.ld16<NT>((uint32_t)(lane * 16));
#pragma unroll
    for (int c = 0; c < 4; c++) w[c] = v[c];
    if constexpr (B == 3) {
      const uint64_t h = t.ld8<NT>((uint32_t)(1024 + lane * 8));
      w[4] = (uint32_t)h;
      w[5] = (uint32_t)(h >> 32);
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
    const int fi = 2 * f + s;
    constexpr uint32_t magic = 0x64006400u;
    if constexpr (B == 2) {
      const uint32_t q = (fi & 1) ? w[fi >> 1] >> 8 : w[fi >> 1];
      p = 2 * j;
      return and_or_b32(q, 0x00030003u << p, magic);
    } else {
      const int P = 4 * fi + j;
      if (P < 30) {
        const int fld = P % 5;
        const uint32_t q = fld < 3 ? w[P / 5] : w[P / 5] >> 9;
        p = 3 * (fld < 3 ? fld : fld - 3);
        return and_or_b32(q, 0x00070007u << p, magic);
      }
      const int d0 = 3 * (P - 30);
      p = 0;
      uint32_t t = and_or_b32(w[d0] >> 15, 0x00010001u, magic);
      t = and_or_b32(w[d0 + 1] >> 14, 0x00020002u, t);
      return and_or_b32(w[d0 + 2] >> 13, 0x00040004u, t);
    }
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
template <> struct WTile<MOE_I5_G32> : WTileB<5> {};
template <> struct WTile<MOE_I6_G32> : WTileB<6> {};
template <> struct WTile<MOE_I7_G32> : WTileB<7> {};
template <> struct WTile<MOE_I8_G32> : WTileB<8> {};

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
