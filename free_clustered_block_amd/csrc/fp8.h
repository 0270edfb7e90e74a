// FP8 (OCP E4M3) operands of the attention's Q.K^T product on gfx950.
//
// The paper's kernel is quantized and is compared with quantized dense
// attention ("ClusterAttention: A training-free speedup of bidirectional
// attention", arXiv 2608.26965 v1 §4.1 "Baselines"); the scheme is not given
// there. Here a group of values (one query row, or 64 consecutive keys of a
// cluster) shares one scale: amax = max |x| over the group, inv =
// fp32(448 / amax) (0 for an all-zero group), code = e4m3(fp32(x * inv))
// rounded to nearest even (v_cvt_pk_fp8_f32), and the dequantized value is
// code * fp32(amax / 448). Products of two codes are exact in fp32, so the
// matrix core returns sum(code_q * code_k) and the logit is that sum times
// s_q * s_k.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operand formats e4m3 (0) and
// scale operands 0 (the unscaled form) computes C[32][32] += A[32][64] *
// B[64][32]: lane l (h = l / 32, r = l % 32) supplies 32 bytes of row r of A
// and 32 bytes of column r of B, the two wave halves holding disjoint parts
// of the contraction, indexed the same way for A and B; C is laid out as in
// the bf16 instruction.
#pragma once

#include "common.h"

namespace ca {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kE4m3Max = 448.0f;

CA_DEV floatx16_t mfma32_fp8(const i32x8_t& a, const i32x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// FP8 value operands of P.V: a block of 32 values of one head dimension shares
// a power-of-two scale 2^e (the OCP microscaling E8M0 block scale, byte
// e + 127), e the smallest integer with amax <= 448 * 2^e (at least -127; 0
// for an all-zero block): with amax = m 2^x, m in [0.5, 1), and 448 = 0.875
// 2^9, e = x - 9 if m <= 0.875 else x - 8. The MFMA applies the scale of
// operand A per row and 32-element block of the contraction (opsel picks the
// byte of the scale register); operand B (the attention weights, <= 256 by
// the lazy running maximum, exact in range) takes scale byte 127 (2^0).
CA_DEV int e8m0_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x;
  const float m = frexpf(amax, &x);
  const int e = m <= 0.875f ? x - 9 : x - 8;
  return e < -127 ? -127 : e;
}

template <int OPSEL_A>
CA_DEV floatx16_t mfma32_fp8_scale_a(const i32x8_t& a, const i32x8_t& b, const floatx16_t& c,
                                     int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL_A, scale_a, 0, 0x7F);
}

// Four values (already in range) as four e4m3 codes, byte i = value i.
CA_DEV uint32_t e4m3_pack4_raw(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

// inv = 448 / amax (0 for amax == 0) and the dequantization scale amax / 448,
// both rounded to nearest in fp32.
CA_DEV float e4m3_inv(float amax) { return amax > 0.0f ? __fdiv_rn(kE4m3Max, amax) : 0.0f; }
CA_DEV float e4m3_scale(float amax) { return __fdiv_rn(amax, kE4m3Max); }

// Four values times inv, as four e4m3 codes (byte i = value i).
CA_DEV uint32_t e4m3_pack4(float x0, float x1, float x2, float x3, float inv) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(x0, inv), __fmul_rn(x1, inv), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(x2, inv), __fmul_rn(x3, inv), w, true);
  return (uint32_t)w;
}

// Eight bf16 values (one 16-byte chunk) times inv, as eight codes.
CA_DEV u32x2_t e4m3_pack_bf16x8(const u32x4_t& v, float inv) {
  u32x2_t r;
  r.x = e4m3_pack4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16),
                   bf16_to_f32(v.y & 0xFFFFu), bf16_to_f32(v.y >> 16), inv);
  r.y = e4m3_pack4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16),
                   bf16_to_f32(v.w & 0xFFFFu), bf16_to_f32(v.w >> 16), inv);
  return r;
}

// Largest magnitude of eight bf16 values: the magnitude bits order like the
// values, so an integer maximum over (bits & 0x7FFF) is exact.
CA_DEV uint32_t amax_bits_bf16x8(const u32x4_t& v, uint32_t m) {
  const uint32_t lo = 0x7FFFu, hi = 0x7FFF0000u;
  m = max(m, max(v.x & lo, (v.x & hi) >> 16));
  m = max(m, max(v.y & lo, (v.y & hi) >> 16));
  m = max(m, max(v.z & lo, (v.z & hi) >> 16));
  m = max(m, max(v.w & lo, (v.w & hi) >> 16));
  return m;
}

}  // namespace ca
