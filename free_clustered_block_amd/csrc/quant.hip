// Group quantization of rows to FP8 (OCP E4M3), the operand format of the
// attention's FP8 Q.K^T variant ("ClusterAttention: A training-free speedup
// of bidirectional attention", arXiv 2608.26965 v1 §4.1 "Baselines": the
// kernel is quantized; the group scheme is the one stated in fp8.h). It uses
// the same amax, scale and code helpers as the attention kernels.
//
// One workgroup of 256 threads per group of `group` consecutive rows: the
// group's largest magnitude by a block reduction, then the codes.
#include <type_traits>

#include "fp8.h"
#include "kernels.h"

namespace ca {

namespace {

CA_DEV float abs_elem(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i] & 0x7FFFu); }
CA_DEV float abs_elem(const float* p, int64_t i) { return fabsf(p[i]); }

template <typename T>
__global__ __launch_bounds__(256) void quantize_rows(const T* X, int64_t rows, int D, int group,
                                                     uint8_t* codes, float* scales) {
  __shared__ float swm[4];
  const int tid = threadIdx.x;
  const int64_t ngroups = (rows + group - 1) / group;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t r0 = g * group;
    const int64_t n = (min((int64_t)group, rows - r0)) * D;   // elements of the group
    const T* src = X + r0 * D;
    uint8_t* dst = codes + r0 * D;
    float m = 0.0f;
    for (int64_t e = tid; e < n; e += 256) m = fmaxf(m, abs_elem(src, e));
    m = wave_max(m);
    __syncthreads();   // the previous group's reads of swm are done
    if ((tid & 63) == 0) swm[tid >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(swm[0], swm[1]), fmaxf(swm[2], swm[3]));
    const float inv = e4m3_inv(amax);
    bool done = false;
    if constexpr (std::is_same<T, uint16_t>::value) {
      if (D % 8 == 0) {   // 16-byte chunks of eight bf16, as the key tiles are written
        const u32x4_t* s8 = reinterpret_cast<const u32x4_t*>(src);
        for (int64_t e = tid; e < n / 8; e += 256)
          *reinterpret_cast<u32x2_t*>(dst + 8 * e) = e4m3_pack_bf16x8(s8[e], inv);
        done = true;
      }
    }
    if (!done)
      for (int64_t e = tid; e < n; e += 256)
        dst[e] = (uint8_t)(e4m3_pack4(load_elem(src, e), 0.0f, 0.0f, 0.0f, inv) & 0xFFu);
    if (tid == 0) scales[g] = e4m3_scale(amax);
  }
}

}  // namespace

void launch_quantize_e4m3(const void* X, int dtype, int64_t rows, int D, int group, uint8_t* codes,
                          float* scales, hipStream_t st) {
  const int64_t ngroups = (rows + group - 1) / group;
  const unsigned grid = (unsigned)(ngroups < 16384 ? ngroups : 16384);
  if (dtype == 0)
    quantize_rows<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)X, rows, D, group, codes, scales);
  else
    quantize_rows<float><<<grid, 256, 0, st>>>((const float*)X, rows, D, group, codes, scales);
}

}  // namespace ca
