// Cluster assignment (paper v1 §3.3): score every query cluster against every
// key cluster by the centroid product qbar . kbar (Eq. 18, the mean logit),
// then keep the top-k key clusters per query cluster (§3.3.2), ties to the
// lower index, written in ascending order.
#include "kernels.h"

namespace ca {

namespace {

constexpr int kTile = 64;
constexpr int kDChunk = 32;

// A[bh][i][j] = sum_d cq[bh][i][d] ck[bh][j][d], summed in increasing d.
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ cq,
                                                     const float* __restrict__ ck, int nq,
                                                     int nk, int D, float* __restrict__ A) {
  __shared__ float sa[kTile][kDChunk + 1];
  __shared__ float sb[kTile][kDChunk + 1];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const float* Q = cq + (int64_t)bh * nq * D;
  const float* K = ck + (int64_t)bh * nk * D;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int d0 = 0; d0 < D; d0 += kDChunk) {
    for (int e = threadIdx.x; e < kTile * kDChunk; e += 256) {
      const int rr = e / kDChunk, dd = e % kDChunk;
      sa[rr][dd] = (i0 + rr < nq) ? Q[(int64_t)(i0 + rr) * D + d0 + dd] : 0.0f;
      sb[rr][dd] = (j0 + rr < nk) ? K[(int64_t)(j0 + rr) * D + d0 + dd] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < kDChunk; ++dd) {
      float av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = sa[ty * 4 + a][dd];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = sb[tx + 16 * b][dd];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = i0 + ty * 4 + a, j = j0 + tx + 16 * b;
      if (i < nq && j < nk) A[((int64_t)bh * nq + i) * nk + j] = acc[a][b];
    }
}

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxKeys = 8192;

// One workgroup per (head, query cluster): radix-select the k smallest
// (~order_key(score), index) pairs, i.e. the k largest scores with ties to the
// lower index, then compact their indices in ascending order.
__global__ __launch_bounds__(kSelThreads) void topk_kernel(const float* __restrict__ A, int nq,
                                                           int nk, int k,
                                                           int32_t* __restrict__ blocks) {
  __shared__ uint32_t skeys[kMaxKeys];
  __shared__ int hist[kSelWaves][256];
  __shared__ int wtot[2][kSelWaves];
  __shared__ uint32_t sel[2];
  const int row = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const float* a = A + ((int64_t)bh * nq + row) * nk;
  for (int i = tid; i < nk; i += kSelThreads) skeys[i] = ~order_key(a[i]);
  __syncthreads();

  uint32_t prefix = 0;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < nk; i += kSelThreads) {
      const uint32_t kk = skeys[i];
      if ((kk & hmask) == (prefix & hmask)) atomicAdd(&hist[w][(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    if (w == 0) {
      int v[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int tot = 0;
        for (int q = 0; q < kSelWaves; ++q) tot += hist[q][4 * l + j];
        v[j] = tot;
        s += tot;
      }
      int inc = s;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, 64);
        if (l >= d) inc += y;
      }
      int before = inc - s;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < want && want <= before + v[j]) {
          sel[0] = (uint32_t)(4 * l + j);
          sel[1] = (uint32_t)before;
        }
        before += v[j];
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    want -= (int)sel[1];
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int eq_take = want;
  int32_t* out = blocks + ((int64_t)bh * nq + row) * k;
  int eq_base = 0, s_base = 0;
  for (int base = 0; base < nk; base += kSelThreads) {
    const int i = base + tid;
    const bool valid = i < nk;
    const uint32_t kk = valid ? skeys[i] : 0xFFFFFFFFu;
    const bool less = valid && kk < kstar;
    const bool eq = valid && kk == kstar;
    uint64_t bal;
    const int eqpre = lane_prefix(eq, &bal);
    if (l == 0) wtot[0][w] = __popcll(bal);
    __syncthreads();
    int eq_w = 0, eq_all = 0;
    for (int q = 0; q < kSelWaves; ++q) {
      if (q < w) eq_w += wtot[0][q];
      eq_all += wtot[0][q];
    }
    const bool take = less || (eq && eq_base + eq_w + eqpre < eq_take);
    const int spre = lane_prefix(take, &bal);
    if (l == 0) wtot[1][w] = __popcll(bal);
    __syncthreads();
    int s_w = 0, s_all = 0;
    for (int q = 0; q < kSelWaves; ++q) {
      if (q < w) s_w += wtot[1][q];
      s_all += wtot[1][q];
    }
    if (take && s_base + s_w + spre < k) out[s_base + s_w + spre] = i;
    eq_base += eq_all;
    s_base += s_all;
    __syncthreads();
  }
}

}  // namespace

void launch_route(const float* cq, const float* ck, int BH, int nq, int nk, int D, int topk,
                  float* scores, int32_t* blocks, hipStream_t st) {
  dim3 gs((nk + kTile - 1) / kTile, (nq + kTile - 1) / kTile, BH);
  scores_kernel<<<gs, 256, 0, st>>>(cq, ck, nq, nk, D, scores);
  dim3 gt(nq, BH);
  topk_kernel<<<gt, kSelThreads, 0, st>>>(scores, nq, nk, topk, blocks);
}

}  // namespace ca
