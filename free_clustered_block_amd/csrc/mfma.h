// CDNA4 (gfx950) matrix-core helpers: v_mfma_f32_32x32x16_bf16.
//
// One instruction computes C[32][32] += A[32][16] * B[16][32] for a wave64.
// Operand layout (lane l, h = l / 32, r = l % 32):
//   A: lane l supplies A[r][8h + e]            for e = 0..7 (bf16x8)
//   B: lane l supplies B[8h + e][r]            for e = 0..7 (bf16x8)
//   C: lane l holds   C[8(i/4) + 4h + i%4][r]  for i = 0..15 (floatx16)
// A and B index the contraction dimension the same way, so any consistent
// relabelling of it gives the same product.
#pragma once

#include "common.h"

namespace ca {

CA_DEV floatx16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the C/D tile held in element i of lane l.
CA_DEV int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

CA_DEV bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

CA_DEV u32x4_t pack8(const float* f) {
  u32x4_t r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + the sum of the eight bf16 values packed in v (v_dot2_f32_bf16 with a
// pair of ones: each pair is added in fp32).
CA_DEV float sum_bf16x8(const u32x4_t& v, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  const bf16x8_t p = __builtin_bit_cast(bf16x8_t, v);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  return acc;
}
CA_DEV floatx16_t zero16() {
  floatx16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

}  // namespace ca
