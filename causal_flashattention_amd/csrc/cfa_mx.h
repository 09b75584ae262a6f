// Block-scaled (MX) encoders on bf16 bit patterns, shared by the operand passes and the MX
// forward kernel (which quantises its own Q rows). Rules and the instruction semantics they
// rest on are stated at the top of mx_quantize.hip.
#pragma once
#include "cfa_device.h"

namespace cfa {

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
typedef __attribute__((ext_vector_type(2))) short s16x2;

__device__ inline uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ inline uint32_t min_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Largest magnitude bit pattern (0..0x7FFF) of the bf16 pairs w[0..n).
template <int N>
__device__ inline uint32_t amax_bits(const uint32_t* w) {
  uint32_t m = w[0] & 0x7FFF7FFFu;
#pragma unroll
  for (int i = 1; i < N; ++i) m = max_u16x2(m, w[i] & 0x7FFF7FFFu);
  return max(m & 0xFFFFu, m >> 16);
}

// Block exponents from the largest magnitude's bf16 bits: floor(log2 amax) - top exponent,
// clamped below at -127 (zero and bf16 subnormal blocks give -127; no finite block reaches 127).
__device__ inline int e4m3_block_exp(uint32_t ab) { return max((int)(ab >> 7) - 135, -127); }
__device__ inline int e2m1_block_exp(uint32_t ab) { return max((int)(ab >> 7) - 129, -127); }

// Four E4M3 codes (little-endian) of the bf16 pairs a, b (elements a.lo, a.hi, b.lo, b.hi) in a
// block with exponent e.
__device__ inline int e4m3_encode4(uint32_t a, uint32_t b, int e) {
  const uint32_t c = ((uint32_t)(e + 135) << 7) | 0x60u;      // bf16 bits of 448·2^e
  const uint32_t cc = c | (c << 16);
  const float s = __builtin_amdgcn_ldexpf(1.f, e);
  const uint32_t ac = min_u16x2(a & 0x7FFF7FFFu, cc) | (a & 0x80008000u);
  const uint32_t bc = min_u16x2(b & 0x7FFF7FFFu, cc) | (b & 0x80008000u);
  // the first conversion writes bits 15:0 and the second bits 31:16, so the first call's
  // pass-through half may hold anything (here the input itself: no register to clear)
  s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2, ac), __builtin_bit_cast(bf16x2, ac),
                                                      s, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, bc), s, true);
  return __builtin_bit_cast(int, r);
}

// max over the four lanes 4k..4k+3 (lane swaps 1 and 2 as DPP quad permutations: no LDS trip)
__device__ inline uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  return v;
}

// c, or the NaN/Inf block's code word k where bad (a select, not a branch)
__device__ inline int bad_or(bool bad, int k, int c) { return bad ? k : c; }

// Eight E2M1 codes (element 2i in the low nibble of byte i) of the bf16 pairs w[0..4).
__device__ inline uint32_t e2m1_encode8(const uint32_t* w, int e) {
  const float s = __builtin_amdgcn_ldexpf(1.f, e);
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, w[0]), s, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[1]), s, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[2]), s, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[3]), s, 3);
  return r;
}

// 6-bit codes (QF 2: E2M3, 3: E3M2) of one whole 32-element block held by one lane (16 bf16 pairs):
// v_cvt_scalef32_pk32_{fp6,bf6}_bf16 divides by 2^e, rounds to nearest even, saturates at the
// format's largest value (7.5 / 28) and packs code i at bits 6i..6i+5 of 192. An in-bounds probe
// over every bf16 pattern (in groups of 32) and block exponents -127..125 matched the software
// encoders of mx_quantize.hip bit for bit.
typedef __attribute__((ext_vector_type(6))) unsigned u32x6;
template <int QF>
__device__ inline int e6_block_exp(uint32_t ab) { return max((int)(ab >> 7) - (QF == 2 ? 129 : 131), -127); }
template <int QF>
__device__ inline u32x6 e6_encode32(const uint32_t* w, int e) {
  typedef __attribute__((ext_vector_type(32))) __bf16 bf16x32;
  typedef __attribute__((ext_vector_type(16))) uint32_t u32x16;
  u32x16 v;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = w[i];
  const bf16x32 x = __builtin_bit_cast(bf16x32, v);
  const float sc = __builtin_amdgcn_ldexpf(1.f, e);
  if constexpr (QF == 2) return __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(x, sc);
  else return __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(x, sc);
}

// maximum over the lane pair (l, l ^ 32) of a non-negative integer (v_permlane32_swap)
__device__ inline uint32_t pair_max32_u(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}

}  // namespace cfa
