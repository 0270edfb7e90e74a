// Peak-rate probes of the matrix cores and of LDS, measured beside the path
// so that roofline fractions can be read against what the chip delivers as
// well as against the published peaks. Not part of the attention path.
#include "kernels.h"
#include "mfma.h"

namespace ca {

namespace {

// Four independent v_mfma_f32_32x32x16_bf16 chains per wave, operands in
// registers, iters rounds. 32768 FLOP per instruction.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* out) {
  const int tid = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + 0.001f * (float)((tid + e) & 7));
    b[e] = (__bf16)(0.5f - 0.001f * (float)((tid * 3 + e) & 7));
  }
  floatx16_t c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  s = wave_sum(s);
  if ((tid & 63) == 0) out[blockIdx.x * 4 + (tid >> 6)] = s;
}

// Conflict-free ds_read_b128 from a 16 KB LDS block: each round, every lane
// reads 8 x 16 bytes at rotating offsets. 1 KB per wave instruction.
__global__ __launch_bounds__(256) void peak_lds_kernel(int iters, float* out) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[4096];
  const int tid = threadIdx.x;
  for (int i = tid; i < 4096; i += 256) buf[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int l = tid & 63;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  int off = (l * 4 + (tid >> 6) * 1024) & 4095;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&buf[(off + k * 256) & 4095]);
      acc.x ^= v.x; acc.y += v.y; acc.z ^= v.z; acc.w += v.w;
    }
    off = (off + 4) & 4095;
  }
  if (l == 0) out[blockIdx.x * 4 + (tid >> 6)] = (float)((acc.x ^ acc.y ^ acc.z ^ acc.w) & 0xFFFF);
}

}  // namespace

void launch_peak_mfma(int blocks, int iters, float* out, hipStream_t st) {
  peak_mfma_kernel<<<blocks, 256, 0, st>>>(iters, out);
}

void launch_peak_lds(int blocks, int iters, float* out, hipStream_t st) {
  peak_lds_kernel<<<blocks, 256, 0, st>>>(iters, out);
}

}  // namespace ca
