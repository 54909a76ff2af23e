// device_common.h -- small device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Two floats -> two bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// The 32x32x16 bf16 MFMA: C[32x32] += A[32x16] * B[16x32].  Lane l supplies
// A row (l % 32), B column (l % 32), K elements 8*(l/32) .. +7; it receives
// C column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4) for accumulator r.
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// A staging tile in LDS: rows of 64 bf16 (128 B) = eight 16-byte chunks; chunk
// c of row r sits at slot c ^ (r & 7), so the 16-byte reads of 8 consecutive
// rows at one K offset hit 8 different bank groups.
__device__ __forceinline__ int lds_a_index(int row, int chunk) {
  return row * 64 + ((chunk ^ (row & 7)) << 3);  // in bf16 elements
}

// Byte n of a dword as a float, one v_cvt_f32_ubyte<n> each (the compiler
// otherwise splits the byte extraction into a separate bit-field extract).
__device__ __forceinline__ float ubyte0_f(uint32_t x) {
  float r;
  asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float ubyte1_f(uint32_t x) {
  float r;
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float ubyte2_f(uint32_t x) {
  float r;
  asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float ubyte3_f(uint32_t x) {
  float r;
  asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Signed byte n of a dword as a float: the SDWA form selects and sign-extends
// the byte inside the convert.
#define MOE_SBYTE_F(N)                                                                     \
  __device__ __forceinline__ float sbyte##N##_f(uint32_t x) {                              \
    float r;                                                                               \
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_" #N \
        : "=v"(r)                                                                          \
        : "v"(x));                                                                         \
    return r;                                                                              \
  }
MOE_SBYTE_F(0)
MOE_SBYTE_F(1)
MOE_SBYTE_F(2)
MOE_SBYTE_F(3)
#undef MOE_SBYTE_F

// (x & m) | o in one instruction (the masks live in registers: gfx9 VOP3
// encodings take no literal operands).
__device__ __forceinline__ uint32_t and_or_b32(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(o));
  return r;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// ---- per-token power-of-two scale of int4-layer activations ---------------
// Gate/up of int4 (and b-bit) layers run fp16 MFMA on x * 2^-e, e per token
// chosen so the row's largest magnitude lies in [2^14, 2^15): every bf16
// value of the row is then exact in fp16 unless it lies 2^28 below that
// largest.  2^e is undone on the fp32 accumulator.

// e for a row whose largest magnitude has float bits mx (e = 0 for an
// all-zero row).
__device__ __forceinline__ int row_fp16_exponent(uint32_t mx) {
  int e = 0;
  if (mx != 0) {
    const int ex = (int)(mx >> 23) - 127;  // floor(log2 max|x|) for normal values
    e = max(ex, -126) - 14;
    e = max(e, -100);
  }
  return e;
}

// Largest |x| of a bf16 row of `pieces` 16-byte pieces, as float bits (finite
// non-negative floats order as integers), by one wave; every lane gets it.
// Each lane loads XB pieces at a time with no condition on the loads (indices
// past the row re-read its last piece), so a batch is in flight at once.
constexpr int XB = 8;  // 16-byte pieces per lane per batch (d <= 4096 in one)
__device__ __forceinline__ uint32_t wave_row_absmax_bf16(const u32x4_t* src, int pieces) {
  const int lane = threadIdx.x & 63;
  uint32_t mx = 0;
  for (int p0 = 0; p0 < pieces; p0 += 64 * XB) {
    u32x4_t v[XB];
#pragma unroll
    for (int j = 0; j < XB; j++) v[j] = src[min(p0 + 64 * j + lane, pieces - 1)];
#pragma unroll
    for (int j = 0; j < XB; j++)
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const uint32_t a = (v[j][w] << 16) & 0x7fffffffu, b = v[j][w] & 0x7fff0000u;
        mx = max(mx, max(a, b));
      }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  return mx;
}

// Two bf16 values (one dword) times 2^-e (`down`, exact) as two fp16 values,
// rounded to nearest even: the fp16 staging of an int4-layer activation pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_scaled(uint32_t v, float down) {
  f16x2_t h = {(_Float16)(bf16_lo(v) * down), (_Float16)(bf16_hi(v) * down)};
  return __builtin_bit_cast(uint32_t, h);
}

// Token row t of x (d bf16 values) as fp16 times 2^-e into x16, 2^e into
// xscale[t], by one wave (the wave's lanes load XB pieces at a time, as in
// wave_row_absmax_bf16; pieces past the row are re-read and not stored).
__device__ __forceinline__ void wave_row_to_f16(int t, int d, const uint16_t* __restrict__ x,
                                                uint16_t* __restrict__ x16,
                                                float* __restrict__ xscale) {
  const int lane = threadIdx.x & 63;
  const u32x4_t* src = (const u32x4_t*)(x + (size_t)t * d);
  const int pieces = d / 8;
  const int e = row_fp16_exponent(wave_row_absmax_bf16(src, pieces));
  const float down = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
  if (lane == 0) xscale[t] = __uint_as_float((uint32_t)(127 + e) << 23);
  u32x4_t* dst = (u32x4_t*)(x16 + (size_t)t * d);
  for (int p0 = 0; p0 < pieces; p0 += 64 * XB) {
    u32x4_t v[XB];
#pragma unroll
    for (int j = 0; j < XB; j++) v[j] = src[min(p0 + 64 * j + lane, pieces - 1)];
#pragma unroll
    for (int j = 0; j < XB; j++) {
      const int p = p0 + 64 * j + lane;
      u32x4_t o;
#pragma unroll
      for (int w = 0; w < 4; w++) o[w] = bf16x2_to_f16x2_scaled(v[j][w], down);
      if (p < pieces) dst[p] = o;
    }
  }
}

// Rows t = w, w + nw, ... (< T) of x to fp16, wave w of nw.
__device__ __forceinline__ void rows_to_f16(int T, int d, const uint16_t* __restrict__ x,
                                            uint16_t* __restrict__ x16,
                                            float* __restrict__ xscale, int w, int nw) {
  for (int t = w; t < T; t += nw) wave_row_to_f16(t, d, x, x16, xscale);
}

}  // namespace moe
