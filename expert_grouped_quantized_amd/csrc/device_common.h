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

}  // namespace moe
