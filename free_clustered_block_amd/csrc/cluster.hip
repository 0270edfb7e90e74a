// Recursive principal-direction splitting of queries and keys (paper v1
// §3.2.1 "Basic recursive splitting", transforms of §3.2.2; the later
// revision's §4.1.1 places the split with radix-select passes).
//
// One tree per (head, tensor); all trees and all nodes of a depth advance
// together, three launches per depth:
//   pddp_dir      one workgroup per node: content-hash subsample, centred
//                 covariance applied implicitly, warm-started power iteration
//                 u <- M C u with the metric M injected (no eigendecomposition);
//   pddp_project  one workgroup per c positions: score = u . x over rows
//                 gathered through the permutation, mapped to ordered uint32;
//   pddp_split    one workgroup per node: 4 x 8-bit LDS radix select of the
//                 rank-t key with a position tie-break, then a stable
//                 partition of the node's permutation slice.
// The node layout depends only on (N, c) and is recomputed on the device, so
// no host synchronisation is needed between levels.
#include "kernels.h"

namespace ca {

namespace {

// ----------------------------------------------------------------------------
// Direction of each node
// ----------------------------------------------------------------------------

template <typename T>
struct DirLds;

template <int D, typename T>
constexpr int dir_cap() {
  // sample rows kept in LDS: 48 KB of row storage
  return (48 * 1024) / (D * (int)sizeof(T));
}

// Row r of the sample (r < m) as float, read from LDS when cached.
template <int D, typename T>
struct SampleRows {
  const T* X;            // token rows of this head and tensor
  const int32_t* list;   // sample token ids
  const float* s;        // per-token scale (queries) or null
  const T* lds;          // [cap][D + pad]
  const float* lds_s;    // [cap]
  int cap, pitch;

  CA_DEV float scale(int r) const {
    if (r < cap) return lds_s[r];
    return s ? s[list[r]] : 1.0f;
  }
  CA_DEV float elem(int r, int j) const {
    if (r < cap) return load_elem(lds, (int64_t)r * pitch + j);
    return load_elem(X, (int64_t)list[r] * D + j);
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void pddp_dir(LevelArgs a) {
  constexpr int CAP = dir_cap<D, T>();
  constexpr int PITCH = D + (sizeof(T) == 2 ? 2 : 1);   // rotate banks between rows
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* srow = reinterpret_cast<T*>(smem);
  float* ss = reinterpret_cast<float*>(smem + (size_t)CAP * PITCH * sizeof(T));
  float* sz = ss + CAP;          // z_r for cached rows
  float* su = sz + CAP;          // u            [D]
  float* su0 = su + D;           // warm start   [D]
  float* sw = su0 + D;           // w            [D]
  float* smean = sw + D;         // sample mean  [D]
  float* sred = smean + D;       // reductions   [16]
  int* scnt = reinterpret_cast<int*>(sred + 16);   // [16]

  const int tree = blockIdx.y, slot = blockIdx.x;
  const int bh = tree >> 1, tensor = tree & 1;
  int off, n;
  if (!node_at(a.N, a.c, a.level, slot, &off, &n) || n <= a.c) return;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const T* X = reinterpret_cast<const T*>(tensor == 0 ? a.Q : a.K) + (int64_t)bh * a.N * D;
  const float* svec = tensor == 0 ? a.s + (int64_t)bh * a.N : nullptr;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N + off;
  const uint64_t* hash = a.hash + (int64_t)tree * a.N;
  int32_t* list = a.sample_buf + (int64_t)tree * a.N + off;
  float* zg = a.zbuf + (int64_t)tree * a.N + off;

  // --- subsample: Bernoulli at rate min(1, a D / n) on the content hash ----
  uint64_t salt = 0;
  salt = chain_step(salt, a.seed);
  salt = chain_step(salt, kDomainSample);
  salt = chain_step(salt, (uint64_t)tensor);
  salt = chain_step(salt, (uint64_t)a.level);
  const uint64_t ad = (uint64_t)a.sample_factor * D;
  const bool take_all = ad >= (uint64_t)n;
  const uint64_t thr = take_all ? 0 : ((ad << 32) / (uint64_t)n);
  int m = 0;
  for (int base = 0; base < n; base += 256) {
    const int i = base + tid;
    bool acc = false;
    int tok = 0;
    if (i < n) {
      tok = perm[i];
      acc = take_all || ((fmix64(hash[tok] ^ salt) >> 32) < thr);
    }
    uint64_t bal;
    const int pre = lane_prefix(acc, &bal);
    if (l == 0) scnt[w] = __popcll(bal);
    __syncthreads();
    int wbase = 0;
    for (int q = 0; q < w; ++q) wbase += scnt[q];
    int tot = 0;
    for (int q = 0; q < 4; ++q) tot += scnt[q];
    if (acc) list[m + wbase + pre] = tok;
    m += tot;
    __syncthreads();
  }
  const int32_t* rows = list;
  if (m < 2) {   // fewer than two sampled rows: use the whole node
    rows = perm;
    m = n;
  }

  // --- cache the first CAP rows in LDS ------------------------------------
  const int mc = m < CAP ? m : CAP;
  for (int e = tid; e < mc * D; e += 256) {
    const int r = e / D, j = e % D;
    srow[r * PITCH + j] = X[(int64_t)rows[r] * D + j];
  }
  for (int r = tid; r < mc; r += 256) ss[r] = svec ? svec[rows[r]] : 1.0f;
  __syncthreads();
  SampleRows<D, T> S{X, rows, svec, srow, ss, CAP, PITCH};

  // --- sample mean ----------------------------------------------------------
  const float inv_m = 1.0f / (float)m;
  if (tid < D) {
    float acc = 0.0f;
    for (int r = 0; r < m; ++r) acc += S.scale(r) * S.elem(r, tid);
    smean[tid] = acc * inv_m;
  }

  // --- warm start: normalise(parent + unit random vector) ------------------
  if (tid < D) {
    uint64_t base = 0;
    base = chain_step(base, a.seed);
    base = chain_step(base, kDomainWarm);
    base = chain_step(base, (uint64_t)bh);
    base = chain_step(base, (uint64_t)tensor);
    base = chain_step(base, (uint64_t)a.level);
    base = chain_step(base, (uint64_t)slot);
    const uint64_t z = fmix64(base + (uint64_t)(tid + 1) * kGolden);
    float rj = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) rj += ((float)((z >> (16 * k)) & 0xFFFFu) + 0.5f) * (1.0f / 65536.0f);
    su0[tid] = rj - 2.0f;
  }
  __syncthreads();
  auto block_sum = [&](float v) -> float {
    v = wave_sum(v);
    __syncthreads();
    if (l == 0) sred[w] = v;
    __syncthreads();
    return sred[0] + sred[1] + sred[2] + sred[3];
  };
  {
    float r = tid < D ? su0[tid] : 0.0f;
    const float nr = sqrtf(block_sum(r * r));
    float rh = r / nr;
    if (a.level > 0) {
      const float* par = a.dir_prev + ((int64_t)tree * (1 << (a.level - 1)) + (slot >> 1)) * D;
      const float sv = tid < D ? par[tid] + rh : 0.0f;
      const float ns = sqrtf(block_sum(sv * sv));
      if (ns > 0.0f) rh = sv / ns;
    }
    if (tid < D) { su0[tid] = rh; su[tid] = rh; }
  }
  __syncthreads();

  // --- power iteration: u <- M C u / |M C u| ------------------------------
  const float* M = (tensor == 0 ? a.Mk : a.Mq) + (int64_t)bh * D * D;
  bool fallback = false;
  for (int it = 0; it < a.power_iters; ++it) {
    // z_r = (x_r - mean) . u
    for (int r = tid; r < m; r += 256) {
      const float sc = S.scale(r);
      float acc = 0.0f;
      for (int jj = 0; jj < D; ++jj) {
        const int j = (jj + r) & (D - 1);
        acc += (sc * S.elem(r, j) - smean[j]) * su[j];
      }
      if (r < CAP) sz[r] = acc; else zg[r] = acc;
    }
    __syncthreads();
    // w = (1/m) sum_r z_r (x_r - mean)
    if (tid < D) {
      float acc = 0.0f;
      for (int r = 0; r < m; ++r) {
        const float zr = r < CAP ? sz[r] : zg[r];
        acc += zr * (S.scale(r) * S.elem(r, tid) - smean[tid]);
      }
      sw[tid] = acc * inv_m;
    }
    __syncthreads();
    // u' = M w
    float un = 0.0f;
    if (tid < D) {
      if (a.transform) {
        float acc = 0.0f;
        for (int k = 0; k < D; ++k) acc += M[(int64_t)k * D + tid] * sw[k];
        un = acc;
      } else {
        un = sw[tid];
      }
    }
    const float nn = block_sum(un * un);
    if (nn == 0.0f) { fallback = true; break; }
    if (tid < D) su[tid] = un / sqrtf(nn);
    __syncthreads();
  }
  __syncthreads();
  float* out = a.dir_cur + ((int64_t)tree * (1 << a.level) + slot) * D;
  if (tid < D) out[tid] = fallback ? su0[tid] : su[tid];
}

template <typename T, int D>
size_t dir_smem() {
  constexpr int CAP = dir_cap<D, T>();
  constexpr int PITCH = D + (sizeof(T) == 2 ? 2 : 1);
  return (size_t)CAP * PITCH * sizeof(T) + (size_t)(2 * CAP + 4 * D + 16) * 4 + 16 * 4;
}

// ----------------------------------------------------------------------------
// Projection of every member of every splitting node
// ----------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void pddp_project(LevelArgs a) {
  constexpr int LPR = 4;                 // lanes per row
  constexpr int EPL = D / LPR;           // elements per lane
  const int tree = blockIdx.y;
  const int bh = tree >> 1, tensor = tree & 1;
  const int p0 = blockIdx.x * a.c;
  int off, n, idx;
  const int depth = node_of(a.N, a.c, a.level, p0, &off, &n, &idx);
  if (depth < a.level || n <= a.c) return;   // inside a leaf

  const int tid = threadIdx.x, q = tid & (LPR - 1);
  const float* u = a.dir_cur + ((int64_t)tree * (1 << a.level) + idx) * D + q * EPL;
  float ur[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ur[e] = u[e];
  const T* X = reinterpret_cast<const T*>(tensor == 0 ? a.Q : a.K) + (int64_t)bh * a.N * D;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N;
  const float* svec = tensor == 0 ? a.s + (int64_t)bh * a.N : nullptr;
  uint32_t* keys = a.keys + (int64_t)tree * a.N;
  const int pend = min(a.N, p0 + a.c);
  for (int pb = p0; pb < pend; pb += 256 / LPR) {
    const int p = pb + tid / LPR;
    float acc = 0.0f;
    int tok = 0;
    if (p < pend) {
      tok = perm[p];
      const T* row = X + (int64_t)tok * D + q * EPL;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int g = 0; g < EPL / 8; ++g) {
          const u32x4_t v = reinterpret_cast<const u32x4_t*>(row)[g];
          const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc += bf16_to_f32((uint16_t)(ws[k] & 0xFFFFu)) * ur[g * 8 + 2 * k];
            acc += bf16_to_f32((uint16_t)(ws[k] >> 16)) * ur[g * 8 + 2 * k + 1];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc += load_elem(row, e) * ur[e];
      }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (p < pend && q == 0) {
      const float score = svec ? svec[tok] * acc : acc;
      keys[p] = order_key(score);
      if (a.trace_score) a.trace_score[(int64_t)tree * a.N + p] = score;
    }
  }
}

// ----------------------------------------------------------------------------
// Radix select + stable partition of every splitting node; leaves are copied.
// ----------------------------------------------------------------------------

constexpr int kSplitThreads = 512;
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kSplitCache = 8192;   // keys kept in LDS

__global__ __launch_bounds__(kSplitThreads) void pddp_split(LevelArgs a) {
  __shared__ uint32_t skeys[kSplitCache];
  __shared__ int hist[kSplitWaves][256];
  __shared__ int wtot[2][kSplitWaves];
  __shared__ uint32_t sel[4];

  const int tree = blockIdx.y, slot = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // walk to the slot; find the segment this slot owns
  int o = 0, m = a.N, depth = 0;
  for (; depth < a.level; ++depth) {
    if (m <= a.c) break;
    const int t = split_size(m, a.c);
    if ((slot >> (a.level - 1 - depth)) & 1) { o += t; m -= t; } else { m = t; }
  }
  const int32_t* pin = a.perm_in + (int64_t)tree * a.N;
  int32_t* pout = a.perm_out + (int64_t)tree * a.N;
  if (depth < a.level || m <= a.c) {
    // leaf: copied once, by the slot whose remaining path bits are all zero
    const int below = a.level - depth;
    if (below > 0 && (slot & ((1 << below) - 1)) != 0) return;
    for (int i = tid; i < m; i += kSplitThreads) pout[o + i] = pin[o + i];
    return;
  }
  const int off = o, n = m;
  const int t = split_size(n, a.c);
  const uint32_t* gkeys = a.keys + (int64_t)tree * a.N + off;
  const bool cached = n <= kSplitCache;
  if (cached)
    for (int i = tid; i < n; i += kSplitThreads) skeys[i] = gkeys[i];
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t { return cached ? skeys[i] : gkeys[i]; };

  uint32_t prefix = 0;
  int want = t;   // 1-based rank still to locate among the candidates
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kSplitWaves * 256; i += kSplitThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < n; i += kSplitThreads) {
      const uint32_t k = key_at(i);
      if ((k & hmask) == (prefix & hmask)) atomicAdd(&hist[w][(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (w == 0) {
      int v[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int tot = 0;
        for (int q = 0; q < kSplitWaves; ++q) tot += hist[q][4 * l + j];
        v[j] = tot;
        s += tot;
      }
      // inclusive scan of the lane totals
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
  const int eq_take = want;   // elements equal to kstar that go left

  int eq_base = 0, left_base = 0;
  for (int base = 0; base < n; base += kSplitThreads) {
    const int i = base + tid;
    const bool valid = i < n;
    uint32_t k = 0;
    int pv = 0;
    if (valid) { k = key_at(i); pv = pin[off + i]; }
    const bool less = valid && k < kstar;
    const bool eq = valid && k == kstar;
    uint64_t bal;
    const int eqpre = lane_prefix(eq, &bal);
    if (l == 0) wtot[0][w] = __popcll(bal);
    __syncthreads();
    int eq_w = 0, eq_all = 0;
    for (int q = 0; q < kSplitWaves; ++q) {
      if (q < w) eq_w += wtot[0][q];
      eq_all += wtot[0][q];
    }
    const int eq_rank = eq_base + eq_w + eqpre;
    const bool left = less || (eq && eq_rank < eq_take);
    const int lpre = lane_prefix(left, &bal);
    if (l == 0) wtot[1][w] = __popcll(bal);
    __syncthreads();
    int l_w = 0, l_all = 0;
    for (int q = 0; q < kSplitWaves; ++q) {
      if (q < w) l_w += wtot[1][q];
      l_all += wtot[1][q];
    }
    const int lrank = left_base + l_w + lpre;
    if (valid) {
      const int dest = left ? off + lrank : off + t + (i - lrank);
      if (dest < off + n) pout[dest] = pv;   // holds by construction; guards the slice
    }
    eq_base += eq_all;
    left_base += l_all;
    __syncthreads();
  }
}

__global__ void perm_init(int32_t* perm, int trees, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)trees * N) perm[i] = (int32_t)(i % N);
}

__global__ void perm_out(const int32_t* perm, int BH, int N, int32_t* pq, int32_t* pk) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)BH * N) return;
  const int64_t bh = i / N, p = i % N;
  pq[i] = perm[(2 * bh) * N + p];
  pk[i] = perm[(2 * bh + 1) * N + p];
}

// Means of the original rows of every cluster; rows summed in position order.
template <typename T, int D>
__global__ __launch_bounds__(256) void centroids_kernel(const T* __restrict__ Q,
                                                        const T* __restrict__ K, int N, int c,
                                                        const int32_t* __restrict__ pq,
                                                        const int32_t* __restrict__ pk,
                                                        float* __restrict__ cq,
                                                        float* __restrict__ ck,
                                                        int32_t* __restrict__ counts) {
  constexpr int G = 256 / D;   // row groups
  __shared__ float part[G][D];
  const int j = blockIdx.x, bh = blockIdx.y, tensor = blockIdx.z;
  const int nc = (N + c - 1) / c;
  const int nj = min(c, N - j * c);
  const T* X = (tensor == 0 ? Q : K) + (int64_t)bh * N * D;
  const int32_t* perm = (tensor == 0 ? pq : pk) + (int64_t)bh * N + (int64_t)j * c;
  const int d = threadIdx.x % D, g = threadIdx.x / D;
  float acc = 0.0f;
  for (int r = g; r < nj; r += G) acc += load_elem(X, (int64_t)perm[r] * D + d);
  part[g][d] = acc;
  __syncthreads();
  if (g == 0) {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < G; ++q) s += part[q][d];
    float* out = (tensor == 0 ? cq : ck) + ((int64_t)bh * nc + j) * D;
    out[d] = s / (float)nj;
    if (d == 0 && tensor == 0 && counts) counts[(int64_t)bh * nc + j] = nj;
  }
}

}  // namespace

void launch_perm_init(int32_t* perm, int trees, int N, hipStream_t st) {
  const int64_t n = (int64_t)trees * N;
  perm_init<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, trees, N);
}

void launch_perm_out(const int32_t* perm, int BH, int N, int32_t* pq, int32_t* pk, hipStream_t st) {
  const int64_t n = (int64_t)BH * N;
  perm_out<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, BH, N, pq, pk);
}

template <typename T, int D>
static void level_impl(const LevelArgs& a, hipStream_t st) {
  const int trees = 2 * a.BH;
  dim3 gslots(1u << a.level, trees);
  pddp_dir<T, D><<<gslots, 256, dir_smem<T, D>(), st>>>(a);
  dim3 gproj((a.N + a.c - 1) / a.c, trees);
  pddp_project<T, D><<<gproj, 256, 0, st>>>(a);
  pddp_split<<<gslots, kSplitThreads, 0, st>>>(a);
}

void launch_level(const LevelArgs& a, hipStream_t st) {
  if (a.dtype == 0) {
    if (a.D == 64) level_impl<uint16_t, 64>(a, st); else level_impl<uint16_t, 128>(a, st);
  } else {
    if (a.D == 64) level_impl<float, 64>(a, st); else level_impl<float, 128>(a, st);
  }
}

void launch_centroids(const void* Q, const void* K, int dtype, int BH, int N, int D, int c,
                      const int32_t* pq, const int32_t* pk, float* cq, float* ck,
                      int32_t* counts, hipStream_t st) {
  dim3 g((N + c - 1) / c, BH, 2);
  if (dtype == 0) {
    const uint16_t* q = (const uint16_t*)Q;
    const uint16_t* k = (const uint16_t*)K;
    if (D == 64) centroids_kernel<uint16_t, 64><<<g, 256, 0, st>>>(q, k, N, c, pq, pk, cq, ck, counts);
    else centroids_kernel<uint16_t, 128><<<g, 256, 0, st>>>(q, k, N, c, pq, pk, cq, ck, counts);
  } else {
    const float* q = (const float*)Q;
    const float* k = (const float*)K;
    if (D == 64) centroids_kernel<float, 64><<<g, 256, 0, st>>>(q, k, N, c, pq, pk, cq, ck, counts);
    else centroids_kernel<float, 128><<<g, 256, 0, st>>>(q, k, N, c, pq, pk, cq, ck, counts);
  }
}

}  // namespace ca
