// Cluster assignment (paper v1 §3.3): score every query cluster against every
// key cluster by the centroid product qbar . kbar (Eq. 18, the mean logit),
// then keep the top-k key clusters per query cluster (§3.3.2), ties to the
// lower index, written in ascending order; or, adaptively, the clusters above
// a histogram cutoff that meets a minimum count and a mass recall.
#include <mutex>

#include "kernels.h"
#include "wave_select.h"

namespace ca {

// Score matrix of ca_route_noalloc: a file-scope device array instead of a
// caller workspace. Every GPU the library runs on holds its own copy until
// the process ends; host code must use the address hipGetSymbolAddress
// returns for the current device, never the array's name (in host code that
// name is only a stand-in for the symbol).
static __device__ __align__(256) float scratch[kRouteScratchFloats];

int route_scratch(float** out, const char** err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = "no usable current HIP device";
    return 1;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = hipGetErrorString(e);
      return 1;
    }
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return 0;
}

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
  // the next d chunk is staged in registers while the current one is in use
  constexpr int EPT = kTile * kDChunk / 256;   // elements per thread and chunk
  float ra[EPT], rb[EPT];
  auto fetch = [&](int d0) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = (int)threadIdx.x + 256 * k, rr = e / kDChunk, dd = e % kDChunk;
      ra[k] = (i0 + rr < nq) ? Q[(int64_t)(i0 + rr) * D + d0 + dd] : 0.0f;
      rb[k] = (j0 + rr < nk) ? K[(int64_t)(j0 + rr) * D + d0 + dd] : 0.0f;
    }
  };
  fetch(0);
  for (int d0 = 0; d0 < D; d0 += kDChunk) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = (int)threadIdx.x + 256 * k, rr = e / kDChunk, dd = e % kDChunk;
      sa[rr][dd] = ra[k];
      sb[rr][dd] = rb[k];
    }
    __syncthreads();
    if (d0 + kDChunk < D) fetch(d0 + kDChunk);
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

// Rows of at most kWaveSelMax key clusters: one wave per (head, query
// cluster), four per workgroup, the one-wave selection of the k smallest
// (~order_key(score), index) pairs; the taken indices are visited in
// ascending order with their rank, which is their output slot.
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ A, int nq, int nk,
                                                        int k, int32_t* __restrict__ blocks) {
  __shared__ int hist[4][256];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w, bh = blockIdx.y;
  if (row >= nq) return;   // the whole wave
  const float* a = A + ((int64_t)bh * nq + row) * nk;
  int32_t* out = blocks + ((int64_t)bh * nq + row) * k;
  wave_select(l, nk, k, [&](int i) { return ~order_key(a[i]); }, hist[w],
              [&](int i, bool take, int rank) {
                if (take && rank < k) out[rank] = i;
              });
}

// ----------------------------------------------------------------------------
// Adaptive selection (v1 §3.3.2 "Selection"; later revision §4.2): per query
// cluster, the key clusters of highest score until both a minimum count and
// an estimated attention-mass recall are reached. Two histogram passes with
// shared edges for the two criteria: 128 bins over [lo, hi], the lower of the
// two cutoff bins refined into 128 sub-bins; the cutoff is the lower edge of
// the lower cutoff sub-bin. A score's bin is key >> 7 and its sub-bin key &
// 127 with key = min(16383, floor(((s - lo) * (128 / (hi - lo))) * 128)) in
// fp32 (round-to-nearest, no contraction). The mass of cluster j is
// n_j exp(tau (s_j - hi)), held as an integer in units of 2^-40 so that sums
// are exact and the passes deterministic; the target is
// floor(recall * total) in double.
// ----------------------------------------------------------------------------

constexpr int kAdaBins = 128;

__device__ __forceinline__ int ada_key(float s, float lo, float scale) {
  const float u = __fmul_rn(__fsub_rn(s, lo), scale);
  const float f = floorf(__fmul_rn(u, (float)kAdaBins));
  return f >= 0.0f ? (int)fminf(f, (float)(kAdaBins * kAdaBins - 1)) : 0;   // NaN -> 0
}

__device__ __forceinline__ uint64_t ada_mass(float s, float hi, float tau, int cnt) {
  const float m = (float)cnt * expf(__fmul_rn(tau, __fsub_rn(s, hi)));
  return (uint64_t)rint((double)m * 0x1p40);
}

// Wave 0: highest bin b with carried + sum over bins >= b reaching thr
// (kAdaBins when the carried total already does, 0 if no bin does). Lane l
// holds bins 2l and 2l + 1; a suffix sum over the lanes gives every bin's
// cumulative total, and since it only grows towards lower bins, the bins
// that reach thr are 0 .. b: b + 1 of them.
template <typename T>
__device__ int ada_cutoff(const T* hist, T carried, T thr) {
  const int l = threadIdx.x & 63;
  if (carried >= thr) return kAdaBins;
  const T h0 = hist[2 * l], h1 = hist[2 * l + 1];
  T suf = h0 + h1;   // becomes the sum over bins >= 2 l
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T y = __shfl_down(suf, d, 64);
    if (l + d < 64) suf += y;
  }
  const T c0 = carried + suf, c1 = carried + suf - h0;   // cumulative at bins 2 l, 2 l + 1
  const int n = __popcll(__ballot(c0 >= thr)) + __popcll(__ballot(c1 >= thr));
  return n > 0 ? n - 1 : 0;
}

__global__ __launch_bounds__(kSelThreads) void adaptive_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ counts, int nq, int nk, float tau,
    double recall, int min_count, int32_t* __restrict__ blocks, int32_t* __restrict__ nsel) {
  __shared__ int skey[kMaxKeys];
  __shared__ int hc[kAdaBins];
  __shared__ unsigned long long hm[kAdaBins];
  __shared__ float sred[2][kSelWaves];
  __shared__ int wtot[kSelWaves];
  __shared__ int sk[4];
  __shared__ unsigned long long smass[2];
  const int row = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const float* a = A + ((int64_t)bh * nq + row) * nk;
  const int32_t* cn = counts + (int64_t)bh * nk;
  int32_t* out = blocks + ((int64_t)bh * nq + row) * nk;

  float lo = INFINITY, hi = -INFINITY;
  for (int i = tid; i < nk; i += kSelThreads) {
    const float v = a[i];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  lo = -wave_max(-lo);
  hi = wave_max(hi);
  if (l == 0) { sred[0][w] = lo; sred[1][w] = hi; }
  __syncthreads();
  lo = sred[0][0]; hi = sred[1][0];
  for (int q = 1; q < kSelWaves; ++q) { lo = fminf(lo, sred[0][q]); hi = fmaxf(hi, sred[1][q]); }

  int kstar = 0;   // every key >= 0: all selected
  if (nk > min_count && hi > lo) {
    const float scale = __fdiv_rn((float)kAdaBins, __fsub_rn(hi, lo));
    // pass 1: coarse bins
    if (tid < kAdaBins) { hc[tid] = 0; hm[tid] = 0ull; }
    __syncthreads();
    for (int i = tid; i < nk; i += kSelThreads) {
      const float v = a[i];
      const int k = ada_key(v, lo, scale);
      skey[i] = k;
      atomicAdd(&hc[k >> 7], 1);
      atomicAdd(&hm[k >> 7], (unsigned long long)ada_mass(v, hi, tau, cn[i]));
    }
    __syncthreads();
    if (w == 0) {
      unsigned long long tm = hm[2 * l] + hm[2 * l + 1];
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) tm += __shfl_xor(tm, d, 64);
      const unsigned long long target = (unsigned long long)floor(recall * (double)tm);
      const int bc = ada_cutoff<int>(hc, 0, min_count);
      const int bm = ada_cutoff<unsigned long long>(hm, 0ull, target);
      const int bs = min(bc, bm);
      // totals of the bins above bs
      int c0 = (2 * l > bs ? hc[2 * l] : 0) + (2 * l + 1 > bs ? hc[2 * l + 1] : 0);
      unsigned long long m0 = (2 * l > bs ? hm[2 * l] : 0ull) + (2 * l + 1 > bs ? hm[2 * l + 1] : 0ull);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        c0 += __shfl_xor(c0, d, 64);
        m0 += __shfl_xor(m0, d, 64);
      }
      if (l == 0) {
        sk[0] = bs;
        sk[1] = c0;
        smass[0] = m0;
        smass[1] = target;
      }
    }
    __syncthreads();
    const int bs = sk[0];
    // pass 2: the sub-bins of bin bs
    if (tid < kAdaBins) { hc[tid] = 0; hm[tid] = 0ull; }
    __syncthreads();
    for (int i = tid; i < nk; i += kSelThreads) {
      const int k = skey[i];
      if ((k >> 7) == bs) {
        atomicAdd(&hc[k & 127], 1);
        atomicAdd(&hm[k & 127], (unsigned long long)ada_mass(a[i], hi, tau, cn[i]));
      }
    }
    __syncthreads();
    if (w == 0) {
      const int fc = ada_cutoff<int>(hc, sk[1], min_count);
      const int fm = ada_cutoff<unsigned long long>(hm, smass[0], smass[1]);
      if (l == 0) sk[2] = bs * kAdaBins + min(fc, fm);
    }
    __syncthreads();
    kstar = sk[2];
  } else {
    for (int i = tid; i < nk; i += kSelThreads) skey[i] = 0;
    __syncthreads();
  }
  // compaction in index order
  int base = 0;
  for (int b0 = 0; b0 < nk; b0 += kSelThreads) {
    const int i = b0 + tid;
    const bool take = i < nk && skey[i] >= kstar;
    uint64_t bal;
    const int pre = lane_prefix(take, &bal);
    if (l == 0) wtot[w] = __popcll(bal);
    __syncthreads();
    int before = 0, all = 0;
    for (int q = 0; q < kSelWaves; ++q) {
      if (q < w) before += wtot[q];
      all += wtot[q];
    }
    if (take) out[base + before + pre] = i;
    base += all;
    __syncthreads();
  }
  for (int i = base + tid; i < nk; i += kSelThreads) out[i] = -1;
  if (tid == 0) nsel[(int64_t)bh * nq + row] = base;
}

}  // namespace

void launch_route_adaptive(const float* cq, const float* ck, const int32_t* counts, int BH, int nq,
                           int nk, int D, float tau, double recall, int min_count, float* scores,
                           int32_t* blocks, int32_t* nsel, hipStream_t st) {
  dim3 gs((nk + kTile - 1) / kTile, (nq + kTile - 1) / kTile, BH);
  scores_kernel<<<gs, 256, 0, st>>>(cq, ck, nq, nk, D, scores);
  dim3 gt(nq, BH);
  adaptive_kernel<<<gt, kSelThreads, 0, st>>>(scores, counts, nq, nk, tau, recall, min_count,
                                               blocks, nsel);
}

void launch_route(const float* cq, const float* ck, int BH, int nq, int nk, int D, int topk,
                  float* scores, int32_t* blocks, hipStream_t st) {
  dim3 gs((nk + kTile - 1) / kTile, (nq + kTile - 1) / kTile, BH);
  scores_kernel<<<gs, 256, 0, st>>>(cq, ck, nq, nk, D, scores);
  if (nk <= kWaveSelMax) {
    dim3 gw((nq + 3) / 4, BH);
    topk_wave_kernel<<<gw, 256, 0, st>>>(scores, nq, nk, topk, blocks);
  } else {
    dim3 gt(nq, BH);
    topk_kernel<<<gt, kSelThreads, 0, st>>>(scores, nq, nk, topk, blocks);
  }
}

}  // namespace ca
