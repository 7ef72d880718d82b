// Device-side types and helpers shared by the gfx950 attention kernels.
//
// Lane layouts used throughout (wave64, checked on gfx950 hardware):
//
//  v_mfma_f32_32x32x16_bf16  A (32x16): lane l holds row l%32, 8 k-values
//                            B (16x32): lane l holds column l%32, 8 k-values
//                            A and B use the same k-to-(lane half, element)
//                            assignment, so any consistent ordering of the
//                            contraction index works.
//                            D (32x32): lane l, register r holds
//                            row 8*(r/4) + 4*(l/32) + r%4, column l%32.
//  v_mfma_f32_16x16x32_bf16  A: lane l holds row l%16; B: column l%16;
//                            D: lane l, register r holds row 4*(l/16) + r,
//                            column l%16.
//  v_mfma_f32_32x32x2_f32    A: lane l holds A[l%32][l/32]; B: B[l/32][l%32];
//                            D as for the 32x32 bf16 form.
//  ds_read_b64_tr_b16        within each group of 16 lanes, lane i receives
//                            element i%4 of the 8 bytes addressed by lanes
//                            4t + i/4, for t = 0..3.  If lane 4t+u points at
//                            row r0+t, column c0+4u of a row-major bf16 tile,
//                            lane i receives column c0+i of rows r0..r0+3.
//  v_permlane32_swap         swaps the upper half of its first operand with
//                            the lower half of its second; with both operands
//                            x, the two results hold x[l] and x[l^32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing 8-byte LDS read (see the layout note above).  The pointer is
// restrict-qualified so that the read carries alias-scope information: the
// compiler's wait insertion then treats it like an ordinary LDS load instead
// of waiting for every outstanding global->LDS copy before it (the kernels
// order those copies against their reads with explicit vmcnt waits and
// barriers).
__device__ __forceinline__ u32x2 lds_read_tr16(const __attribute__((address_space(3))) u16* __restrict__ p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_read_tr16(const u16* __restrict__ p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Byte-transposing 8-byte LDS read (ds_read_b64_tr_b8).  Within each group of
// 16 lanes, lane i receives byte i % 8 of the 8-byte chunks addressed by
// lanes 2t + i / 8, t = 0..7, in that order: if lane 2t + u points at bytes
// 8u .. 8u+7 of a row R_t, lane i gets column i of rows R_0 .. R_7.
// Restrict-qualified for the same reason as lds_read_tr16.
__device__ __forceinline__ u32x2 lds_read_tr8(const __attribute__((address_space(3))) uint8_t* __restrict__ p) {
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Eight E4M3 codes (byte k of the pair = element k) to eight bf16 values.
// Every E4M3 value is a bf16 value, so the conversion is exact; the scale
// operand of the conversion is 1.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

// max(x[l], x[l^32]) and x[l] + x[l^32] across the two wave halves.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ u16 f2bf(float x) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
// the same as one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace miattn
