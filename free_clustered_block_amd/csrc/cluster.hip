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
#include <algorithm>
#include <utility>

#include "kernels.h"
#include "mfma.h"
#include "wave_select.h"

namespace ca {

namespace {

// ----------------------------------------------------------------------------
// Node subsample (Bernoulli at rate min(1, a D / n) on the content hash):
// one workgroup per c positions writes its sampled tokens, compacted in
// position order, at the chunk's own offset, and their count. A node's sample
// is the concatenation of its chunks' lists, so it is independent of the
// launch order and of the number of workgroups.
// ----------------------------------------------------------------------------

constexpr int kSampleSpan = 1024;   // positions per workgroup (a multiple of every c)

__global__ __launch_bounds__(256) void pddp_sample(LevelArgs a) {
  __shared__ int wcnt[4];
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base;
  const int tensor = tree & 1;
  const int tid = threadIdx.x, w = tid >> 6;
  uint64_t salt = 0;
  salt = chain_step(salt, a.seed);
  salt = chain_step(salt, kDomainSample);
  salt = chain_step(salt, (uint64_t)tensor);
  salt = chain_step(salt, (uint64_t)a.level);
  const uint64_t ad = (uint64_t)a.sample_factor * a.D;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N;
  const uint64_t* hpos = a.hpos_in + (int64_t)tree * a.N;
  // four slabs of 256 positions; a chunk of c <= 256 positions lies in one slab
  int tok[4];
  bool flag[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = blockIdx.x * kSampleSpan + k * 256 + tid;
    flag[k] = false;
    tok[k] = 0;
    int off, n, idx;
    const int depth = p < a.N ? node_of(a.N, a.c, a.level, p, &off, &n, &idx) : -1;
    if (depth == a.level && n > a.c) {
      tok[k] = perm[p];
      const bool take_all = ad >= (uint64_t)n;
      const uint64_t thr = take_all ? 0 : ((ad << 32) / (uint64_t)n);
      flag[k] = take_all || ((fmix64(hpos[p] ^ salt) >> 32) < thr);
    }
  }
  const int waves_per_chunk = a.c >> 6;   // c in {64, 128, 256}
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = blockIdx.x * kSampleSpan + k * 256 + tid;
    uint64_t bal;
    const int pre = lane_prefix(flag[k], &bal);
    if ((tid & 63) == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    const int w0 = (w / waves_per_chunk) * waves_per_chunk;   // first wave of this chunk
    int base = 0, tot = 0;
    for (int q = w0; q < w0 + waves_per_chunk; ++q) {
      if (q < w) base += wcnt[q];
      tot += wcnt[q];
    }
    const int chunk = p >> __builtin_ctz((unsigned)a.c);   // c is a power of two
    if (flag[k]) a.sample_buf[(int64_t)tree * a.N + (int64_t)chunk * a.c + base + pre] = tok[k];
    if (p < a.N && (p & (a.c - 1)) == 0) a.chunk_cnt[(int64_t)tree * a.nchunks + chunk] = tot;
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// Direction of each node: p power iterations u <- M C u / |M C u| from the
// warm start, C the centred covariance of the node's sample, M the metric of
// the tensor (injected; no root matrix). One workgroup of 256 threads per
// node; the first CAP sample rows live in LDS, M lives in registers.
// ----------------------------------------------------------------------------

template <int D, typename T>
struct DirCfg {
  static constexpr int TPR = 256 / D;          // threads per row (z) and per M row
  static constexpr int EPT = D / TPR;          // elements per thread
  static constexpr int G = 256 / D;            // row groups for column sums
  static constexpr int PITCH = D + 16 / (int)sizeof(T);   // padded row (elements)
  static constexpr int CAP = (sizeof(T) == 2 ? 56 * 1024 : 96 * 1024) / (PITCH * (int)sizeof(T));
  static constexpr size_t row_bytes = (size_t)CAP * PITCH * sizeof(T);
  // floats after the rows: s[CAP], z[CAP], mean[D], u[D], w[D], u0[D], part[G][D], red[16]
  // without the chunk prefix array, whose length depends on the level
  static constexpr size_t smem = row_bytes + (size_t)(2 * CAP + 4 * D + G * D + 16) * 4 + 16 * 4;
};

template <typename T>
CA_DEV void load_vec(const T* p, float* out, int n) {
  for (int e = 0; e < n; ++e) out[e] = load_elem(p, e);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pddp_dir(LevelArgs a) {
  using Cfg = DirCfg<D, T>;
  constexpr int TPR = Cfg::TPR, EPT = Cfg::EPT, G = Cfg::G, PITCH = Cfg::PITCH, CAP = Cfg::CAP;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* srow = reinterpret_cast<T*>(smem);
  float* ss = reinterpret_cast<float*>(smem + Cfg::row_bytes);
  float* sz = ss + CAP;
  float* smean = sz + CAP;
  float* su = smean + D;
  float* sw = su + D;
  float* su0 = sw + D;
  float* spart = su0 + D;          // [G][D]
  float* sred = spart + G * D;     // [16]
  int* spre = reinterpret_cast<int*>(sred + 16 + 16);   // chunk prefix sums [nch + 1]

  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, slot = blockIdx.x;
  const int bh = tree >> 1, tensor = tree & 1;
  int off, n;
  if (!node_at(a.N, a.c, a.level, slot, &off, &n) || n <= a.c) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const T* X = reinterpret_cast<const T*>(tensor == 0 ? a.Q : a.K) + (int64_t)(tensor == 0 ? bh : bh / a.kvg) * a.N * D;
  const float* svec = tensor == 0 ? a.s + (int64_t)bh * a.N : nullptr;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N + off;
  int32_t* stok = a.zbuf_tok + (int64_t)tree * a.N + off;   // the node's sample tokens

  auto block_sum = [&](float v) -> float {
    v = wave_sum(v);
    __syncthreads();
    if (l == 0) sred[w] = v;
    __syncthreads();
    return sred[0] + sred[1] + sred[2] + sred[3];
  };

  // --- gather the sample: prefix over the node's chunk counts ---------------
  const int ch0 = off / a.c;
  const int nch = (n + a.c - 1) / a.c;
  const int32_t* cnt = a.chunk_cnt + (int64_t)tree * a.nchunks + ch0;
  {
    // per-thread contiguous groups, then a block scan of the group totals
    const int per = (nch + 255) / 256;
    const int g0 = tid * per;
    int gs = 0;
    for (int k = 0; k < per; ++k)
      if (g0 + k < nch) gs += cnt[g0 + k];
    // block exclusive scan of gs
    int inc = gs;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d, 64);
      if (l >= d) inc += y;
    }
    if (l == 63) reinterpret_cast<int*>(sred)[w] = inc;
    __syncthreads();
    int wb = 0;
    for (int q = 0; q < w; ++q) wb += reinterpret_cast<int*>(sred)[q];
    int run = wb + inc - gs;
    for (int k = 0; k < per; ++k)
      if (g0 + k < nch) { spre[g0 + k] = run; run += cnt[g0 + k]; }
    if (tid == 255) spre[nch] = run;
    __syncthreads();
  }
  int m = spre[nch];
  const bool whole = m < 2;     // fewer than two sampled rows: the whole node
  if (whole) m = n;
  __syncthreads();
  const int32_t* lists = a.sample_buf + (int64_t)tree * a.N;
  for (int r = tid; r < m; r += 256) {
    int tok;
    if (whole) {
      tok = perm[r];
    } else {
      int lo = 0, hi = nch - 1;     // last chunk k with spre[k] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (spre[mid] <= r) lo = mid; else hi = mid - 1;
      }
      tok = lists[(int64_t)(ch0 + lo) * a.c + (r - spre[lo])];
    }
    stok[r] = tok;
    if (r < CAP) {
      constexpr int NG = D * (int)sizeof(T) / 16;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(X + (int64_t)tok * D);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(srow + r * PITCH);
      u32x4_t v[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) v[g] = src[g];
#pragma unroll
      for (int g = 0; g < NG; ++g) dst[g] = v[g];
      ss[r] = svec ? svec[tok] : 1.0f;
    }
  }
  // M slice into registers: row jm, columns [qm EPT, (qm+1) EPT)
  const int jm = tid / TPR, qm = tid % TPR;
  const float* M = (tensor == 0 ? a.Mk : a.Mq) + (int64_t)bh * D * D;
  float mreg[EPT];
  if (a.transform) {
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(M + (int64_t)jm * D + qm * EPT + e);
      mreg[e] = v[0]; mreg[e + 1] = v[1]; mreg[e + 2] = v[2]; mreg[e + 3] = v[3];
    }
  }
  __syncthreads();

  // Rows r < mc live in LDS, rows r >= mc (only when the sample exceeds CAP)
  // are read from global memory; the two ranges run as separate loops so that
  // every load has a definite address space.
  const int mc = m < CAP ? m : CAP;
  const int64_t zoff = (int64_t)tree * a.N + off;

  // --- sample mean (column j summed in row order by group, then groups) -----
  const int jc = tid % D, gc = tid / D;
  {
    float acc = 0.0f;
    int r = gc;
#pragma unroll 4
    for (; r < mc; r += G) acc += ss[r] * load_elem(srow, (int64_t)r * PITCH + jc);
    for (; r < m; r += G) {
      const int tok = stok[r];
      acc += (svec ? svec[tok] : 1.0f) * load_elem(X, (int64_t)tok * D + jc);
    }
    spart[gc * D + jc] = acc;
    __syncthreads();
    if (tid < D) {
      float s = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) s += spart[g * D + tid];
      smean[tid] = s / (float)m;
    }
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
  {
    const float r = tid < D ? su0[tid] : 0.0f;
    const float nr = sqrtf(block_sum(r * r));
    float rh = r / nr;
    if (a.level > 0) {
      const float* par = a.dir_prev + ((int64_t)tree * a.node_slots + (slot >> 1)) * D;
      const float sv = tid < D ? par[tid] + rh : 0.0f;
      const float ns = sqrtf(block_sum(sv * sv));
      if (ns > 0.0f) rh = sv / ns;
    }
    if (tid < D) { su0[tid] = rh; su[tid] = rh; }
  }
  __syncthreads();

  // per-thread slices of u and of the mean for the row dots
  const int qz = tid % TPR;
  float mz[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) mz[e] = smean[qz * EPT + e];
  const float mcol = smean[jc];
  const float inv_m = 1.0f / (float)m;

  bool fallback = false;
  for (int it = 0; it < a.power_iters; ++it) {
    float uz[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) uz[e] = su[qz * EPT + e];
    // z_r = (s_r x_r - mean) . u : TPR threads per row, four partial sums.
    // y_r = s_r z_r is kept for w, and Z = sum_r z_r per row group.
    float zpart = 0.0f;
    for (int rb = 0; rb < m; rb += 256 / TPR) {
      const int r = rb + tid / TPR;
      float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      float sr = 1.0f;
      if (r < mc) {
        sr = ss[r];
        const T* row = srow + r * PITCH + qz * EPT;
#pragma unroll
        for (int e = 0; e < EPT; ++e) a4[e & 3] = fmaf(fmaf(sr, load_elem(row, e), -mz[e]), uz[e], a4[e & 3]);
      } else if (r < m) {
        const int tok = stok[r];
        sr = svec ? svec[tok] : 1.0f;
        const T* row = X + (int64_t)tok * D + qz * EPT;
#pragma unroll
        for (int e = 0; e < EPT; ++e) a4[e & 3] = fmaf(fmaf(sr, load_elem(row, e), -mz[e]), uz[e], a4[e & 3]);
      }
      float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
      if (qz == 0 && r < m) {
        zpart += acc;
        if (r < mc) sz[r] = acc * sr;
        else a.zbuf[zoff + r] = acc * sr;
      }
    }
    {
      // Z = sum_r z_r over the block (rows are owned by the qz == 0 lanes)
      const float zsum = block_sum(zpart);
      // w_j = (1/m) sum_r z_r (s_r x_rj - mean_j) = (1/m)(sum_r y_r x_rj - mean_j Z),
      // column j by row group gc with four partial sums; the G groups are added
      // when w is read below
      float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
      int r = gc;
      for (; r + 3 * G < mc; r += 4 * G) {
        a0 = fmaf(sz[r], load_elem(srow, (int64_t)r * PITCH + jc), a0);
        a1 = fmaf(sz[r + G], load_elem(srow, (int64_t)(r + G) * PITCH + jc), a1);
        a2 = fmaf(sz[r + 2 * G], load_elem(srow, (int64_t)(r + 2 * G) * PITCH + jc), a2);
        a3 = fmaf(sz[r + 3 * G], load_elem(srow, (int64_t)(r + 3 * G) * PITCH + jc), a3);
      }
      for (; r < mc; r += G) a0 = fmaf(sz[r], load_elem(srow, (int64_t)r * PITCH + jc), a0);
      for (; r < m; r += G) a1 = fmaf(a.zbuf[zoff + r], load_elem(X, (int64_t)stok[r] * D + jc), a1);
      float acc = (a0 + a1) + (a2 + a3);
      if (gc == 0) acc -= mcol * zsum;
      spart[gc * D + jc] = acc * inv_m;
    }
    __syncthreads();
    // u'_j = sum_k M[j][k] w_k : TPR threads per row of M
    float un;
    if (a.transform) {
      float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float wk = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) wk += spart[g * D + qm * EPT + e];
        a4[e & 3] = fmaf(mreg[e], wk, a4[e & 3]);
      }
      float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
      un = acc;
    } else {
      un = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) un += spart[g * D + jm];
    }
    const float contrib = qm == 0 ? un * un : 0.0f;
    const float nn = block_sum(contrib);
    if (nn == 0.0f) { fallback = true; break; }
    if (qm == 0) su[jm] = un / sqrtf(nn);
    __syncthreads();
  }
  __syncthreads();
  float* out = a.dir_cur + ((int64_t)tree * a.node_slots + slot) * D;
  if (tid < D) {
    const float v = fallback ? su0[tid] : su[tid];
    out[tid] = v;
    if (a.trace_dir) a.trace_dir[((int64_t)tree * a.trace_slots + slot) * D + tid] = v;
  }
}

// ----------------------------------------------------------------------------
// Diagonalized splitting (v1 §3.2.1 "Diagonalized recursive splitting"; later
// revision §4.1.1). Every vector was rotated once into its tree's
// principal-component basis (Y = coordinates x . a_j). A node splits along
// the coordinate of highest population variance over its sample (the lowest
// index on ties): thread (j, g) sums y_j and y_j^2 (fp64) over sample rows g,
// g + G, ...; the projection is then the coordinate itself.
// ----------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void pddp_dir_y(LevelArgs a) {
  constexpr int G = 256 / D;
  __shared__ double sp1[G * D], sp2[G * D];
  __shared__ int sred[16];
  extern __shared__ int spre[];   // [nch + 1]
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, slot = blockIdx.x;
  int off, n;
  if (!node_at(a.N, a.c, a.level, slot, &off, &n) || n <= a.c) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N + off;
  int32_t* stok = a.zbuf_tok + (int64_t)tree * a.N + off;
  const int ch0 = off / a.c;
  const int nch = (n + a.c - 1) / a.c;
  const int32_t* cnt = a.chunk_cnt + (int64_t)tree * a.nchunks + ch0;
  {
    const int per = (nch + 255) / 256;
    const int g0 = tid * per;
    int gs = 0;
    for (int k = 0; k < per; ++k)
      if (g0 + k < nch) gs += cnt[g0 + k];
    int inc = gs;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d, 64);
      if (l >= d) inc += y;
    }
    if (l == 63) sred[w] = inc;
    __syncthreads();
    int wb = 0;
    for (int q = 0; q < w; ++q) wb += sred[q];
    int run = wb + inc - gs;
    for (int k = 0; k < per; ++k)
      if (g0 + k < nch) { spre[g0 + k] = run; run += cnt[g0 + k]; }
    if (tid == 255) spre[nch] = run;
    __syncthreads();
  }
  int m = spre[nch];
  const bool whole = m < 2;     // fewer than two sampled rows: the whole node
  if (whole) m = n;
  const int32_t* lists = a.sample_buf + (int64_t)tree * a.N;
  for (int r = tid; r < m; r += 256) {
    int tok;
    if (whole) {
      tok = perm[r];
    } else {
      int lo = 0, hi = nch - 1;     // last chunk k with spre[k] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (spre[mid] <= r) lo = mid; else hi = mid - 1;
      }
      tok = lists[(int64_t)(ch0 + lo) * a.c + (r - spre[lo])];
    }
    stok[r] = tok;
  }
  __syncthreads();
  const int jc = tid % D, gc = tid / D;
  const float* Yt = a.Y + (int64_t)tree * a.N * D + jc;
  double s1 = 0.0, s2 = 0.0;
  int r = gc;
  for (; r + 3 * G < m; r += 4 * G) {
    float y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) y[u] = Yt[(int64_t)stok[r + u * G] * D];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s1 += (double)y[u];
      s2 = fma((double)y[u], (double)y[u], s2);
    }
  }
  for (; r < m; r += G) {
    const float y = Yt[(int64_t)stok[r] * D];
    s1 += (double)y;
    s2 = fma((double)y, (double)y, s2);
  }
  sp1[gc * D + jc] = s1;
  sp2[gc * D + jc] = s2;
  __syncthreads();
  if (tid < D) {
    double t1 = 0.0, t2 = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) { t1 += sp1[g * D + tid]; t2 += sp2[g * D + tid]; }
    const double mean = t1 / (double)m;
    sp1[tid] = t2 / (double)m - mean * mean;   // population variance of coordinate tid
  }
  __syncthreads();
  if (tid == 0) {
    int jb = 0;
    double best = sp1[0];
    for (int j = 1; j < D; ++j)
      if (sp1[j] > best) { best = sp1[j]; jb = j; }
    sred[0] = jb;
    a.jsel[(int64_t)tree * a.node_slots + slot] = jb;
  }
  __syncthreads();
  const int jb = sred[0];
  float* out = a.dir_cur + ((int64_t)tree * a.node_slots + slot) * D;
  if (tid < D) {
    const float v = a.basis[((int64_t)tree * D + jb) * D + tid];
    out[tid] = v;
    if (a.trace_dir) a.trace_dir[((int64_t)tree * a.trace_slots + slot) * D + tid] = v;
  }
}

// Projection of diagonalized splitting: the chosen coordinate of each member.
__global__ __launch_bounds__(256) void pddp_project_y(LevelArgs a) {
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base;
  const int p0 = blockIdx.x * a.c;
  int off, n, idx;
  const int depth = node_of(a.N, a.c, a.level, p0, &off, &n, &idx);
  if (depth < a.level || n <= a.c) return;   // inside a leaf
  const int j = a.jsel[(int64_t)tree * a.node_slots + idx];
  const int p = p0 + (int)threadIdx.x;
  if (p >= min(a.N, p0 + a.c)) return;
  const int tok = a.perm_in[(int64_t)tree * a.N + p];
  const float score = a.Y[((int64_t)tree * a.N + tok) * a.D + j];
  a.keys[(int64_t)tree * a.N + p] = order_key(score);
  if (a.trace_score) a.trace_score[(int64_t)tree * a.N + p] = score;
}

// LDS of pddp_dir at a level: fixed part + chunk prefix sums of the largest node
template <typename T, int D>
size_t dir_smem(int N, int c, int level) {
  const int64_t nmax = ((int64_t)N >> level) + 2 * (int64_t)c;   // bounds every node at the level
  const int64_t nch = (nmax + c - 1) / c;
  return DirCfg<D, T>::smem + (size_t)(nch + 2) * 4;
}

// ----------------------------------------------------------------------------
// Direction of each node, bf16 rows: the sample's Gram matrix S = sum_r x_r x_r^T
// is formed on the matrix cores (bf16 products are exact in the fp32
// accumulator; a query row x = s q enters as q (s^2 q) with s^2 q split into
// three bf16 parts), centred C = S/m - xbar xbar^T, and the p power iterations
// u <- M C u / |M C u| then run as two d x d matrix-vector products on
// registers. Wave w of the D/32 waves owns columns [32w, 32w + 32) of C and of
// M, both held in the MFMA accumulator layout (C and M are symmetric, so a
// column strip also serves as a row strip). The sample is gathered 128 rows at
// a time in one round trip and stored transposed (dimension-major) in LDS.
// ----------------------------------------------------------------------------

// Matrix-vector step of the power iteration with the vector broadcast across
// lanes instead of re-read from LDS by every lane. The 16 lanes of a DPP row
// (one lane half) need the same 64 vector entries; lane j of the row holds
// entries 32 (j >> 2) + 8 (j & 3) + 4 h + 0..3, and row_newbcast:k hands lane
// k's four values to the whole row, fused into the multiply-add.
template <int K>
CA_DEV void fmac_row_bcast(float& acc, float u, float c) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc)
               : "v"(u), "v"(c), "i"(K));
}
// t4[e] += sum over k of m[4 k + e] * (entry e of row lane k's vector values)
template <int... K>
CA_DEV void matvec_row_bcast(float (&t4)[4], const floatx4_t& uv, const float* m,
                             std::integer_sequence<int, K...>) {
  ((fmac_row_bcast<K>(t4[0], uv[0], m[4 * K]), fmac_row_bcast<K>(t4[1], uv[1], m[4 * K + 1]),
    fmac_row_bcast<K>(t4[2], uv[2], m[4 * K + 2]), fmac_row_bcast<K>(t4[3], uv[3], m[4 * K + 3])),
   ...);
}

template <int D, int SCR = 160>
struct DirMma {
  static constexpr int NW = D / 32;          // waves; wave w owns columns [32w, 32w + 32)
  static constexpr int NT = 64 * NW;         // threads
  static constexpr int RT = D / 32;          // 32-row tiles of C per column strip
  static constexpr int SC = SCR;             // sample rows per gather round (the sample
                                             // averages a D rows; 160 covers it at +3 sd)
  static_assert(SC % 32 == 0, "whole row pairs per thread and round");
  static constexpr int RPT = SC / 16;        // rows per thread and round
  static constexpr int XP = SC + 8;          // padded transposed row (bf16): 16 k + 4 dwords
                                             // apart, so 16 lanes' 16-byte reads hit
                                             // distinct banks
  static constexpr int TOKCAP = 4 * SC;      // sample tokens kept in LDS (whole rounds)
};
// Rows per gather round of a launch: the top levels (few nodes, latency bound)
// take a whole sample in one round; the levels with many nodes, which launch
// per tensor, gather fewer rows a round, which needs fewer registers in
// flight: at D = 128 three waves per SIMD for query trees as well as key
// trees (96 and 128 rows), at D = 64 four (64 and 96 rows).
template <int D, int TS>
constexpr int dir_rows_per_round() {
  return TS < 0 ? 160 : D == 64 ? (TS == 0 ? 64 : 96) : (TS == 0 ? 96 : 128);
}

// TS: the trees of the launch are query trees only (0), key trees only (1),
// or both (-1: tensor = tree & 1). Key rows enter the Gram matrix as they
// are, which needs fewer registers than the three-term query split: the
// key-only version runs three workgroups per CU.
template <int D, int TS>
__global__ __launch_bounds__(DirMma<D>::NT) __attribute__((amdgpu_waves_per_eu(TS < 0 ? 2 : D == 64 ? 4 : 3)))
void pddp_dir_mma(LevelArgs a) {
  using Cf = DirMma<D, dir_rows_per_round<D, TS>()>;
  constexpr int NW = Cf::NW, NT = Cf::NT, RT = Cf::RT, SC = Cf::SC, XP = Cf::XP, RPT = Cf::RPT;
  constexpr int TOKCAP = Cf::TOKCAP;
  __shared__ __attribute__((aligned(16))) uint16_t xt[D][XP];
  __shared__ __attribute__((aligned(16))) float s2c[SC];
  __shared__ int tokl[TOKCAP];
  __shared__ __attribute__((aligned(16))) float xbar[D];
  __shared__ __attribute__((aligned(16))) float su0[D];
  __shared__ __attribute__((aligned(16))) float tbuf[D];
  __shared__ __attribute__((aligned(16))) float vbuf[2][D];   // by iteration parity
  __shared__ float nred[2][NW];                               // |v|^2 per wave, by parity
  __shared__ float red[3][NW];
  __shared__ int ired[NW];
  extern __shared__ int spre[];              // chunk prefix sums [nch + 1]

  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, slot = blockIdx.x;
  const int bh = tree >> 1;
  const int tensor = TS >= 0 ? TS : (tree & 1);
  int off, n;
  if (!node_at(a.N, a.c, a.level, slot, &off, &n) || n <= a.c) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, h = l >> 5;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(tensor == 0 ? a.Q : a.K) + (int64_t)(tensor == 0 ? bh : bh / a.kvg) * a.N * D;
  const float* svec = tensor == 0 ? a.s + (int64_t)bh * a.N : nullptr;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N + off;
  int32_t* stok = a.zbuf_tok + (int64_t)tree * a.N + off;

  // warm start: component j of the random vector and of the parent direction
  float rj = 0.0f, pj = 0.0f;
  if (tid < D) {
    if (a.level > 0)
      pj = a.dir_prev[((int64_t)tree * a.node_slots + (slot >> 1)) * D + tid];
    uint64_t base = 0;
    base = chain_step(base, a.seed);
    base = chain_step(base, kDomainWarm);
    base = chain_step(base, (uint64_t)bh);
    base = chain_step(base, (uint64_t)tensor);
    base = chain_step(base, (uint64_t)a.level);
    base = chain_step(base, (uint64_t)slot);
    const uint64_t z = fmix64(base + (uint64_t)(tid + 1) * kGolden);
#pragma unroll
    for (int k = 0; k < 4; ++k) rj += ((float)((z >> (16 * k)) & 0xFFFFu) + 0.5f) * (1.0f / 65536.0f);
    rj -= 2.0f;
  }

  // Sample size. Chunk-list mode: prefix over the node's chunk counts (lists
  // written by pddp_sample). Inline mode (nodes of at most 32 NT members, so
  // a thread's positions fit one 32-bit mask): thread tid tests the content hashes of positions
  // [tid per, tid per + per) itself, so the sample comes out in position
  // order, as the concatenated chunk lists would.
  const bool inl = a.sample_inline != 0;
  const int ch0 = off / a.c;
  const int nch = (n + a.c - 1) / a.c;
  const int32_t* cnt = a.chunk_cnt + (int64_t)tree * a.nchunks + ch0;
  const int per = inl ? (n + NT - 1) / NT : (nch + NT - 1) / NT;
  const int g0 = tid * per;
  int gs = 0;
  uint32_t sbits = 0;   // inline mode: sampled positions g0 + k of this thread
  int ptok[4] = {0, 0, 0, 0};   // inline mode, per <= 4: their tokens, read with the hashes
  if (inl) {
    uint64_t salt = 0;
    salt = chain_step(salt, a.seed);
    salt = chain_step(salt, kDomainSample);
    salt = chain_step(salt, (uint64_t)tensor);
    salt = chain_step(salt, (uint64_t)a.level);
    const uint64_t ad = (uint64_t)a.sample_factor * D;
    const bool take_all = ad >= (uint64_t)n;
    const uint64_t thr = take_all ? 0 : ((ad << 32) / (uint64_t)n);
    const uint64_t* hpos = a.hpos_in + (int64_t)tree * a.N + off;
    if (per <= 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < per && g0 + k < n) ptok[k] = perm[g0 + k];
    }
    for (int k = 0; k < per; ++k)
      if (g0 + k < n && (take_all || (fmix64(hpos[g0 + k] ^ salt) >> 32) < thr)) sbits |= 1u << k;
    gs = __popc(sbits);
  } else {
    for (int k = 0; k < per; ++k)
      if (g0 + k < nch) gs += cnt[g0 + k];
  }
  {
    const float srr = wave_sum(rj * rj), srp = wave_sum(rj * pj), spp = wave_sum(pj * pj);
    if (l == 0) { red[0][w] = srr; red[1][w] = srp; red[2][w] = spp; }
  }
  int inc = gs;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (l >= d) inc += y;
  }
  if (l == 63) ired[w] = inc;
  __syncthreads();
  int srun = 0;   // inline mode: sample rows before this thread's positions
  {
    int run = inc - gs;
    for (int q = 0; q < w; ++q) run += ired[q];
    if (inl) {
      srun = run;
      if (tid == NT - 1) spre[0] = run + gs;
    } else {
      for (int k = 0; k < per; ++k)
        if (g0 + k < nch) { spre[g0 + k] = run; run += cnt[g0 + k]; }
      if (tid == NT - 1) spre[nch] = run;
    }
    // u0 = normalise(parent + r / |r|), or r / |r| at the root
    float srr = 0.0f, srp = 0.0f, spp = 0.0f;
#pragma unroll
    for (int q = 0; q < NW; ++q) { srr += red[0][q]; srp += red[1][q]; spp += red[2][q]; }
    const float nr = sqrtf(srr);
    float u0 = rj / nr;
    if (a.level > 0) {
      const float ns = sqrtf(spp + 2.0f * (srp / nr) + srr / (nr * nr));
      if (ns > 0.0f) u0 = (pj + rj / nr) / ns;
    }
    if (tid < D) su0[tid] = u0;
  }
  __syncthreads();
  int m = spre[inl ? 0 : nch];
  const bool whole = m < 2;     // fewer than two sampled rows: the whole node
  if (whole) m = n;
  if (inl && !whole) {
    // this thread's sampled positions, in order, at rows srun, srun + 1, ...
    for (uint32_t b = sbits; b; b &= b - 1) {
      const int k = __builtin_ctz(b);
      int tok;
      if (per <= 4) {
        tok = ptok[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) tok = k == q ? ptok[q] : tok;
      } else {
        tok = perm[g0 + k];
      }
      if (srun < TOKCAP) tokl[srun] = tok; else stok[srun] = tok;
      ++srun;
    }
  } else {
    const int32_t* lists = a.sample_buf + (int64_t)tree * a.N;
    for (int rr = tid; rr < m; rr += NT) {
      int tok;
      if (whole) {
        tok = perm[rr];
      } else {
        int lo = 0, hi = nch - 1;     // last chunk k with spre[k] <= rr
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (spre[mid] <= rr) lo = mid; else hi = mid - 1;
        }
        tok = lists[(int64_t)(ch0 + lo) * a.c + (rr - spre[lo])];
      }
      if (rr < TOKCAP) tokl[rr] = tok; else stok[rr] = tok;
    }
  }
  __syncthreads();

  // --- Gram matrix of the sample on the matrix cores -------------------------
  // thread (rp, g) gathers rows 32 j + 2 rp + {0, 1} (j < RPT/2) of a round, dims [8g, 8g + 8)
  const int rp = tid & 15, g = tid >> 4;
  float msum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) msum[e] = 0.0f;
  floatx16_t acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = zero16();
  // metric M[32 rt + c_row(i, h)][32 w + r], packed per lane by the metric pass
  u32x4_t mv[RT * 4];

  for (int base = 0;; base += SC) {
    // sample tokens of the round: LDS for the first TOKCAP rows (whole rounds)
    int tk[RPT];
    if (base < TOKCAP) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int row = base + 32 * (q >> 1) + 2 * rp + (q & 1);
        tk[q] = row < m ? tokl[row] : -1;
      }
    } else {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int row = base + 32 * (q >> 1) + 2 * rp + (q & 1);
        tk[q] = row < m ? __builtin_nontemporal_load(stok + row) : -1;
      }
    }
    u32x4_t v[RPT];
    float sv[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      v[q] = u32x4_t{0u, 0u, 0u, 0u};
      sv[q] = 0.0f;
      if (tk[q] >= 0) {
        v[q] = *reinterpret_cast<const u32x4_t*>(X + (int64_t)tk[q] * D + 8 * g);
        sv[q] = svec ? svec[tk[q]] : 1.0f;
      }
    }
    if (base > 0) __syncthreads();   // the previous round's operand reads are done
#pragma unroll
    for (int j = 0; j < RPT / 2; ++j) {
      const uint32_t a0[4] = {v[2 * j].x, v[2 * j].y, v[2 * j].z, v[2 * j].w};
      const uint32_t a1[4] = {v[2 * j + 1].x, v[2 * j + 1].y, v[2 * j + 1].z, v[2 * j + 1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t x0 = (a0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const uint32_t x1 = (a1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        *reinterpret_cast<uint32_t*>(&xt[8 * g + e][32 * j + 2 * rp]) = x0 | (x1 << 16);
        msum[e] = fmaf(sv[2 * j], bf16_to_f32((uint16_t)x0), msum[e]);
        msum[e] = fmaf(sv[2 * j + 1], bf16_to_f32((uint16_t)x1), msum[e]);
      }
      if (g == 0) {
        s2c[32 * j + 2 * rp] = sv[2 * j] * sv[2 * j];
        s2c[32 * j + 2 * rp + 1] = sv[2 * j + 1] * sv[2 * j + 1];
      }
    }
    const bool last = base + SC >= m;
    __syncthreads();
    const int nks = min(SC, m - base + 15) >> 4;   // 16-row steps holding sample rows
    for (int ks = 0; ks < nks; ++ks) {
      const int k0 = 16 * ks + 8 * h;
      const u32x4_t bw = *reinterpret_cast<const u32x4_t*>(&xt[32 * w + r][k0]);
      if (TS == 1 || (TS < 0 && tensor == 1)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const u32x4_t aw = *reinterpret_cast<const u32x4_t*>(&xt[32 * rt + r][k0]);
          acc[rt] = mfma32(as_bf16x8(aw), as_bf16x8(bw), acc[rt]);
        }
      } else {
        // B = s^2 x as hi + mid + lo bf16 parts (exact to fp32 rounding)
        const floatx4_t sq0 = *reinterpret_cast<const floatx4_t*>(&s2c[k0]);
        const floatx4_t sq1 = *reinterpret_cast<const floatx4_t*>(&s2c[k0 + 4]);
        const float sq[8] = {sq0[0], sq0[1], sq0[2], sq0[3], sq1[0], sq1[1], sq1[2], sq1[3]};
        const uint32_t bb[4] = {bw.x, bw.y, bw.z, bw.w};
        float bh_[8], bm_[8], bl_[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float b = bf16_to_f32((uint16_t)((bb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu)) * sq[e];
          const float hi = (float)(__bf16)b;
          const float rem = b - hi;
          const float mid = (float)(__bf16)rem;
          bh_[e] = hi;
          bm_[e] = mid;
          bl_[e] = rem - mid;
        }
        const bf16x8_t ph = as_bf16x8(pack8(bh_)), pm = as_bf16x8(pack8(bm_)), pl = as_bf16x8(pack8(bl_));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8_t aw = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&xt[32 * rt + r][k0]));
          acc[rt] = mfma32(aw, ph, acc[rt]);
          acc[rt] = mfma32(aw, pm, acc[rt]);
          acc[rt] = mfma32(aw, pl, acc[rt]);
        }
      }
    }
    if (last) break;
  }
  if (a.transform) {   // in flight while the mean and C are formed
    const u32x4_t* mp = reinterpret_cast<const u32x4_t*>(a.Mpk + ((int64_t)tree * D * D) +
                                                         (int64_t)(w * 64 + l) * (RT * 16));
#pragma unroll
    for (int k = 0; k < RT * 4; ++k) mv[k] = mp[k];
  }
  // sample mean: the 16 lanes of a dimension group hold all row pairs
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = msum[e];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
    msum[e] = v;
  }
  const float inv_m = 1.0f / (float)m;
  if (rp == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) xbar[8 * g + e] = msum[e] * inv_m;
  }
  __syncthreads();

  // C = S / m - xbar xbar^T in place
  {
    const float xc = xbar[32 * w + r];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4_t xb = *reinterpret_cast<const floatx4_t*>(&xbar[32 * rt + 8 * q + 4 * h]);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[rt][4 * q + k] = fmaf(acc[rt][4 * q + k], inv_m, -xb[k] * xc);
      }
  }
  float mr[RT * 16];
#pragma unroll
  for (int k = 0; k < RT * 4; ++k) {
    mr[4 * k] = __uint_as_float(mv[k].x);
    mr[4 * k + 1] = __uint_as_float(mv[k].y);
    mr[4 * k + 2] = __uint_as_float(mv[k].z);
    mr[4 * k + 3] = __uint_as_float(mv[k].w);
  }

  // --- power iterations -------------------------------------------------------
  // Iteration it reads v of iteration it - 1 (the warm start first) once and
  // forms t = C v / |v|; |v|^2 is the sum, in wave order, of the per-wave
  // sums of squares its writers left beside it. v and those sums are double
  // buffered by iteration parity: a buffer is rewritten two iterations later,
  // after every wave has passed the barrier that follows its last read.
  bool fallback = false;
  float inv_norm = 1.0f;
  int last = 0;   // buffer holding the final v
  // vector entries this lane holds for its DPP row (lanes past RT * 4 repeat row lane 0's)
  const int j16 = (l & 15) < RT * 4 ? (l & 15) : 0;
  const int vsel = 32 * (j16 >> 2) + 8 * (j16 & 3) + 4 * h;
  for (int it = 0;; ++it) {
    if (it > 0) {
      float nn = 0.0f;
#pragma unroll
      for (int q = 0; q < NW; ++q) nn += nred[(it - 1) & 1][q];
      if (nn == 0.0f) { fallback = true; break; }
      inv_norm = 1.0f / sqrtf(nn);
      if (it == a.power_iters) { last = (it - 1) & 1; break; }
    }
    const float* usrc = it == 0 ? su0 : vbuf[(it - 1) & 1];
    const floatx4_t uv = *reinterpret_cast<const floatx4_t*>(&usrc[vsel]);
    float t4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    {
      float cf[RT * 16];   // the C strip in matvec order: element 4 k + e
#pragma unroll
      for (int k = 0; k < RT * 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) cf[4 * k + e] = acc[k >> 2][4 * (k & 3) + e];
      matvec_row_bcast(t4, uv, cf, std::make_integer_sequence<int, RT * 4>{});
    }
    float tp = (t4[0] + t4[1]) + (t4[2] + t4[3]);
    tp = sum_halves(tp);
    if (it > 0) tp *= inv_norm;
    float vp = tp;
    if (a.transform) {
      if (h == 0) tbuf[32 * w + r] = tp;
      __syncthreads();
      const floatx4_t tv = *reinterpret_cast<const floatx4_t*>(&tbuf[vsel]);
      float v4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      matvec_row_bcast(v4, tv, mr, std::make_integer_sequence<int, RT * 4>{});
      vp = (v4[0] + v4[1]) + (v4[2] + v4[3]);
      vp = sum_halves(vp);
    }
    // both lane halves hold v[32 w + r]: the first half's squares are the wave's share
    const float sq = wave_sum(h == 0 ? vp * vp : 0.0f);
    if (h == 0) vbuf[it & 1][32 * w + r] = vp;
    if (l == 0) nred[it & 1][w] = sq;
    __syncthreads();
  }
  float* out = a.dir_cur + ((int64_t)tree * a.node_slots + slot) * D;
  if (tid < D) {
    const float v = fallback ? su0[tid] : vbuf[last][tid] * inv_norm;
    out[tid] = v;
    if (a.trace_dir) a.trace_dir[((int64_t)tree * a.trace_slots + slot) * D + tid] = v;
  }
}

// ----------------------------------------------------------------------------
// Projection of every member of every splitting node
// ----------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void pddp_project(LevelArgs a) {
  // bf16: 8 lanes per row (each load instruction takes whole 128-byte lines)
  // and two rows per lane group with both rows' loads in flight together;
  // fp32: 4 lanes per row, one row at a time
  constexpr bool BF = sizeof(T) == 2;
  constexpr int LPR = BF ? 8 : 4;        // lanes per row
  constexpr int EPL = D / LPR;           // elements per lane
  constexpr int RPG = BF ? 2 : 1;        // rows per lane group and pass
  constexpr int RPP = 256 / LPR;         // lane groups per workgroup
  // Trees in reverse order on odd levels: the trees the previous level read
  // last are read first, while they are still in the last-level cache.
  const int ty = (a.level & 1) ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int tree = ty * a.tree_step + a.tree_base;
  const int bh = tree >> 1, tensor = tree & 1;
  const int p0 = blockIdx.x * a.c;
  int off, n, idx;
  const int depth = node_of(a.N, a.c, a.level, p0, &off, &n, &idx);
  if (depth < a.level || n <= a.c) return;   // inside a leaf

  const int tid = threadIdx.x, q = tid & (LPR - 1);
  const float* u = a.dir_cur + ((int64_t)tree * a.node_slots + idx) * D + q * EPL;
  float ur[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ur[e] = u[e];
  const T* X = reinterpret_cast<const T*>(tensor == 0 ? a.Q : a.K) + (int64_t)(tensor == 0 ? bh : bh / a.kvg) * a.N * D;
  const int32_t* perm = a.perm_in + (int64_t)tree * a.N;
  const float* svec = tensor == 0 ? a.s + (int64_t)bh * a.N : nullptr;
  uint32_t* keys = a.keys + (int64_t)tree * a.N;
  const int pend = min(a.N, p0 + a.c);
  for (int pb = p0; pb < pend; pb += RPG * RPP) {
    int tok[RPG];
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
      const int p = pb + k * RPP + tid / LPR;
      tok[k] = p < pend ? perm[p] : -1;
    }
    float acc[RPG];
    float sc[RPG];
    if constexpr (BF) {
      u32x4_t v[RPG][EPL / 8];
#pragma unroll
      for (int k = 0; k < RPG; ++k) {
        sc[k] = 1.0f;
        if (tok[k] >= 0) {
          const u32x4_t* row = reinterpret_cast<const u32x4_t*>(X + (int64_t)tok[k] * D + q * EPL);
#pragma unroll
          for (int g = 0; g < EPL / 8; ++g) v[k][g] = row[g];
          if (svec) sc[k] = svec[tok[k]];
        }
      }
#pragma unroll
      for (int k = 0; k < RPG; ++k) {
        acc[k] = 0.0f;
        if (tok[k] >= 0) {
#pragma unroll
          for (int g = 0; g < EPL / 8; ++g) {
            const uint32_t ws[4] = {v[k][g].x, v[k][g].y, v[k][g].z, v[k][g].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[k] += bf16_to_f32((uint16_t)(ws[e] & 0xFFFFu)) * ur[g * 8 + 2 * e];
              acc[k] += bf16_to_f32((uint16_t)(ws[e] >> 16)) * ur[g * 8 + 2 * e + 1];
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < RPG; ++k) {
        acc[k] = 0.0f;
        sc[k] = 1.0f;
        if (tok[k] >= 0) {
          const T* row = X + (int64_t)tok[k] * D + q * EPL;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[k] += load_elem(row, e) * ur[e];
          if (svec) sc[k] = svec[tok[k]];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) acc[k] += __shfl_xor(acc[k], o, 64);
      const int p = pb + k * RPP + tid / LPR;
      if (tok[k] >= 0 && q == 0) {
        const float score = svec ? sc[k] * acc[k] : acc[k];
        keys[p] = order_key(score);
        if (a.trace_score) a.trace_score[(int64_t)tree * a.N + p] = score;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Radix select + stable partition of every splitting node; leaves are copied.
// ----------------------------------------------------------------------------

constexpr int kSplitThreads = 512;          // threads per node below the top levels
constexpr int kSplitThreadsTop = 1024;      // threads per node at the two top levels
constexpr int kSplitCacheMax = 32768;        // keys kept in LDS at most (128 KiB)

CA_DEV int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Split of one node: the members are ordered by (key, position), strictly;
// the first t go left and the rest right, both keeping position order (a
// stable partition). The token's content hash moves with it.
template <int NT>
__global__ __launch_bounds__(NT) void pddp_split(LevelArgs a) {
  constexpr int NW = NT / 64;
  extern __shared__ __attribute__((aligned(16))) uint32_t skeys[];   // a.split_cache keys
  __shared__ int hist[NW][256];
  __shared__ int wtot[2][NW];
  __shared__ uint32_t sel[4];

  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, slot = blockIdx.x;
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
  const uint64_t* hin = a.hpos_in + (int64_t)tree * a.N;
  uint64_t* hout = a.hpos_out + (int64_t)tree * a.N;
  if (depth < a.level || m <= a.c) {
    // leaf: copied once, by the slot whose remaining path bits are all zero
    const int below = a.level - depth;
    if (below > 0 && (slot & ((1 << below) - 1)) != 0) return;
    for (int i = tid; i < m; i += NT) {
      pout[o + i] = pin[o + i];
      hout[o + i] = hin[o + i];
    }
    return;
  }
  const int off = o, n = m;
  const int t = split_size(n, a.c);
  const uint32_t* gkeys = a.keys + (int64_t)tree * a.N + off;

  // radix select of the rank-t key over LDS histograms, 8-bit digits from the
  // highest bit in which the node's keys differ (the bits above it are common
  // to every key and would put every member in one bucket)
  const bool cached = n <= a.split_cache;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  {
    // LB loads in flight per thread (one round trip per LB keys, not per key)
    constexpr int LB = 16;
    for (int i0 = tid; i0 < n; i0 += LB * NT) {
      uint32_t kv[LB];
#pragma unroll
      for (int b = 0; b < LB; ++b) {
        const int i = i0 + b * NT;
        kv[b] = i < n ? gkeys[i] : 0u;
      }
#pragma unroll
      for (int b = 0; b < LB; ++b) {
        const int i = i0 + b * NT;
        if (i < n) {
          if (cached) skeys[i] = kv[b];
          kmin = min(kmin, kv[b]);
          kmax = max(kmax, kv[b]);
        }
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
  }
  if (l == 0) { wtot[0][w] = (int)kmin; wtot[1][w] = (int)kmax; }
  __syncthreads();
  kmin = (uint32_t)wtot[0][0];
  kmax = (uint32_t)wtot[1][0];
  for (int q = 1; q < NW; ++q) {
    kmin = min(kmin, (uint32_t)wtot[0][q]);
    kmax = max(kmax, (uint32_t)wtot[1][q]);
  }
  auto key_at = [&](int i) -> uint32_t { return cached ? skeys[i] : gkeys[i]; };

  const uint32_t diff = kmin ^ kmax;
  const int hb = diff ? 31 - __builtin_clz(diff) : -1;   // highest differing bit
  uint32_t prefix = hb < 0 ? kmin : (hb == 31 ? 0u : kmin & (0xFFFFFFFFu << (hb + 1)));
  int want = t;   // 1-based rank still to locate among the candidates
  for (int hi = hb; hi >= 0;) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - lo)) - 1u;
    const uint32_t hmask = hi == 31 ? 0u : (0xFFFFFFFFu << (hi + 1));
    __syncthreads();   // the previous round's reads of hist and sel are done
    for (int i = tid; i < NW * 256; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll 8
    for (int i = tid; i < n; i += NT) {
      const uint32_t k = key_at(i);
      if ((k & hmask) == (prefix & hmask)) atomicAdd(&hist[w][(k >> lo) & dmask], 1);
    }
    __syncthreads();
    if (w == 0) {
      int v[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int tot = 0;
        for (int q = 0; q < NW; ++q) tot += hist[q][4 * l + j];
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
    prefix |= sel[0] << lo;
    want -= (int)sel[1];
    hi = lo - 1;
  }
  __syncthreads();
  const uint32_t kstar = prefix;
  const int eq_take = want;   // members equal to kstar that go left (lowest positions)

  // stable partition: wave w owns a contiguous region of positions; the
  // regions' counts give each wave its starting ranks, then each wave walks
  // its region 64 members at a time with ballot prefixes
  const int per_w = (n + NW - 1) / NW;
  const int r0 = min(n, w * per_w), r1 = min(n, r0 + per_w);
  int cl = 0, ce = 0;
#pragma unroll 8
  for (int i = r0 + l; i < r1; i += 64) {
    const uint32_t k = key_at(i);
    cl += k < kstar;
    ce += k == kstar;
  }
  cl = wave_sum_int(cl);
  ce = wave_sum_int(ce);
  if (l == 0) { wtot[0][w] = cl; wtot[1][w] = ce; }
  __syncthreads();
  int lb = 0, eb = 0;
  for (int q = 0; q < w; ++q) { lb += wtot[0][q]; eb += wtot[1][q]; }
  int erun = eb;                        // equal members before the current step
  int lrun = lb + min(eb, eq_take);     // left members before the current step
  constexpr int BATCH = 8;   // 64-member steps whose loads are issued together
  for (int base = r0; base < r1; base += 64 * BATCH) {
    uint32_t k[BATCH];
    int pv[BATCH];
    uint64_t hv[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + 64 * b + l;
      k[b] = 0u; pv[b] = 0; hv[b] = 0;
      if (i < r1) { k[b] = key_at(i); pv[b] = pin[off + i]; hv[b] = hin[off + i]; }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + 64 * b + l;
      const bool valid = i < r1;
      const bool less = valid && k[b] < kstar;
      const bool eq = valid && k[b] == kstar;
      uint64_t bal_e, bal_l;
      const int eqpre = lane_prefix(eq, &bal_e);
      const bool left = less || (eq && erun + eqpre < eq_take);
      const int lpre = lane_prefix(left, &bal_l);
      const int lrank = lrun + lpre;
      if (valid) {
        const int dest = left ? off + lrank : off + t + (i - lrank);
        if (dest < off + n) {   // holds by construction; guards the slice
          pout[dest] = pv[b];
          hout[dest] = hv[b];
        }
      }
      erun += __popcll(bal_e);
      lrun += __popcll(bal_l);
    }
  }
}

// ----------------------------------------------------------------------------
// Wide split of the levels whose nodes are too large for one workgroup to
// move quickly (a node of 2^18 members read through one CU several times):
// every node's positions are cut into chunks of kWideChunk, one workgroup per
// chunk. The same selection as pddp_split (the rank-t key by 8-bit radix
// digits from the highest bit in which the node's keys differ, position
// tie-break), with the node's digit histogram summed from per-chunk LDS
// histograms by integer atomics (exact, order-free) and each digit picked by
// one small workgroup per node; then per-chunk counts and a stable scatter
// whose starting ranks are the counts of the node's earlier chunks.
// Per node the workspace holds: [0] kmin, [1] kmax, [2] prefix, [3] want
// (rank still to locate), [4] hi (top bit of the next digit, -1 when done),
// then 256 histogram words; per chunk two counts (less, equal).
// ----------------------------------------------------------------------------

constexpr int kWideChunk = 4096;               // positions per workgroup
constexpr int kWideNode = 65536;               // levels whose largest node is this big go wide
constexpr int kWideSlots = 8;                  // ... and have at most this many node slots
constexpr int kWideState = 8 + 256;            // words of per-node state

// node of slot `slot` at the level: (o, m, depth) as in the split kernels
CA_DEV void wide_node(const LevelArgs& a, int slot, int* o, int* m, int* depth) {
  int oo = 0, mm = a.N, d = 0;
  for (; d < a.level; ++d) {
    if (mm <= a.c) break;
    const int t = split_size(mm, a.c);
    if ((slot >> (a.level - 1 - d)) & 1) { oo += t; mm -= t; } else { mm = t; }
  }
  *o = oo; *m = mm; *depth = d;
}

CA_DEV int32_t* wide_state(const LevelArgs& a, int tree, int slot) {
  return a.wide + ((int64_t)tree * kWideSlots + slot) * kWideState;
}
CA_DEV int32_t* wide_counts(const LevelArgs& a, int tree, int slot, int chunk) {
  return a.wide + (int64_t)2 * a.BH * kWideSlots * kWideState +
         (((int64_t)tree * kWideSlots + slot) * ((a.N + kWideChunk - 1) / kWideChunk) + chunk) * 2;
}

// grid (slots * cpn, trees): per chunk of a splitting node, min and max key
__global__ __launch_bounds__(256) void wide_minmax(LevelArgs a) {
  __shared__ uint32_t red[2][4];
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base;
  const int slot = blockIdx.x / a.wide_cpn, chunk = blockIdx.x % a.wide_cpn;
  int o, n, depth;
  wide_node(a, slot, &o, &n, &depth);
  if (depth < a.level || n <= a.c || chunk * kWideChunk >= n) return;
  const uint32_t* keys = a.keys + (int64_t)tree * a.N + o;
  const int i0 = chunk * kWideChunk, i1 = min(n, i0 + kWideChunk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = i0 + tid; i < i1; i += 256) { const uint32_t k = keys[i]; kmin = min(kmin, k); kmax = max(kmax, k); }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
  }
  if (l == 0) { red[0][w] = kmin; red[1][w] = kmax; }
  __syncthreads();
  if (tid == 0) {
    for (int q = 1; q < 4; ++q) { kmin = min(kmin, red[0][q]); kmax = max(kmax, red[1][q]); }
    int32_t* st = wide_state(a, tree, slot);
    atomicMin(reinterpret_cast<unsigned int*>(&st[0]), kmin);
    atomicMax(reinterpret_cast<unsigned int*>(&st[1]), kmax);
  }
}

// grid (slots, trees): state of each splitting node before the first digit
// (mode 0: reset min/max and histogram; mode 1: digits from the min/max)
__global__ __launch_bounds__(256) void wide_init(LevelArgs a, int mode) {
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, slot = blockIdx.x;
  int o, n, depth;
  wide_node(a, slot, &o, &n, &depth);
  if (depth < a.level || n <= a.c) return;
  int32_t* st = wide_state(a, tree, slot);
  if (mode == 0) {
    if (threadIdx.x == 0) { st[0] = (int32_t)0xFFFFFFFFu; st[1] = 0; }
    for (int i = threadIdx.x; i < 256; i += 256) st[8 + i] = 0;
    return;
  }
  if (threadIdx.x != 0) return;
  const uint32_t kmin = (uint32_t)st[0], kmax = (uint32_t)st[1];
  const uint32_t diff = kmin ^ kmax;
  const int hb = diff ? 31 - __builtin_clz(diff) : -1;   // highest differing bit
  st[2] = (int32_t)(hb < 0 ? kmin : (hb == 31 ? 0u : kmin & (0xFFFFFFFFu << (hb + 1))));
  st[3] = split_size(n, a.c);
  st[4] = hb;
}

// grid (slots * cpn, trees): the chunk's histogram of the current digit over
// the keys that share the prefix, added to the node's histogram
__global__ __launch_bounds__(256) void wide_hist(LevelArgs a) {
  __shared__ int hist[4][256];
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base;
  const int slot = blockIdx.x / a.wide_cpn, chunk = blockIdx.x % a.wide_cpn;
  int o, n, depth;
  wide_node(a, slot, &o, &n, &depth);
  if (depth < a.level || n <= a.c || chunk * kWideChunk >= n) return;
  int32_t* st = wide_state(a, tree, slot);
  const int hi = st[4];
  if (hi < 0) return;   // uniform: the node's rank-t key is known
  const int lo = hi >= 7 ? hi - 7 : 0;
  const uint32_t dmask = (2u << (hi - lo)) - 1u;
  const uint32_t hmask = hi == 31 ? 0u : (0xFFFFFFFFu << (hi + 1));
  const uint32_t prefix = (uint32_t)st[2];
  const int tid = threadIdx.x, w = tid >> 6;
  for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
  __syncthreads();
  const uint32_t* keys = a.keys + (int64_t)tree * a.N + o;
  const int i0 = chunk * kWideChunk, i1 = min(n, i0 + kWideChunk);
#pragma unroll 4
  for (int i = i0 + tid; i < i1; i += 256) {
    const uint32_t k = keys[i];
    if ((k & hmask) == (prefix & hmask)) atomicAdd(&hist[w][(k >> lo) & dmask], 1);
  }
  __syncthreads();
  const int v = hist[0][tid] + hist[1][tid] + hist[2][tid] + hist[3][tid];
  if (v) atomicAdd(&st[8 + tid], v);
}

// grid (slots, trees), 64 threads: the bucket that holds rank `want`, then the
// next digit; the histogram is cleared for it
__global__ __launch_bounds__(64) void wide_pick(LevelArgs a) {
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, slot = blockIdx.x;
  int o, n, depth;
  wide_node(a, slot, &o, &n, &depth);
  if (depth < a.level || n <= a.c) return;
  int32_t* st = wide_state(a, tree, slot);
  const int hi = st[4];
  if (hi < 0) return;
  const int lo = hi >= 7 ? hi - 7 : 0;
  const int l = threadIdx.x;
  const int want = st[3];
  int v[4], s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[j] = st[8 + 4 * l + j]; s += v[j]; }
  int inc = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (l >= d) inc += y;
  }
  int before = inc - s, bsel = 0, bbefore = 0;
  bool mine = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (before < want && want <= before + v[j]) { mine = true; bsel = 4 * l + j; bbefore = before; }
    before += v[j];
  }
  const uint64_t owner = __ballot(mine);
  const int src = owner ? __builtin_ctzll(owner) : 0;   // one lane owns rank `want`
  bsel = __shfl(bsel, src, 64);
  bbefore = __shfl(bbefore, src, 64);
#pragma unroll
  for (int j = 0; j < 4; ++j) st[8 + 4 * l + j] = 0;
  if (l == 0) {
    st[2] = (int32_t)((uint32_t)st[2] | ((uint32_t)bsel << lo));
    st[3] = want - bbefore;
    st[4] = lo - 1;
  }
}

// grid (slots * cpn, trees): members of the chunk below and equal to the
// node's rank-t key
__global__ __launch_bounds__(256) void wide_count(LevelArgs a) {
  __shared__ int red[2][4];
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base;
  const int slot = blockIdx.x / a.wide_cpn, chunk = blockIdx.x % a.wide_cpn;
  int o, n, depth;
  wide_node(a, slot, &o, &n, &depth);
  if (depth < a.level || n <= a.c || chunk * kWideChunk >= n) return;
  const uint32_t kstar = (uint32_t)wide_state(a, tree, slot)[2];
  const uint32_t* keys = a.keys + (int64_t)tree * a.N + o;
  const int i0 = chunk * kWideChunk, i1 = min(n, i0 + kWideChunk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int cl = 0, ce = 0;
#pragma unroll 4
  for (int i = i0 + tid; i < i1; i += 256) {
    const uint32_t k = keys[i];
    cl += k < kstar;
    ce += k == kstar;
  }
  cl = wave_sum_int(cl);
  ce = wave_sum_int(ce);
  if (l == 0) { red[0][w] = cl; red[1][w] = ce; }
  __syncthreads();
  if (tid == 0) {
    int32_t* cc = wide_counts(a, tree, slot, chunk);
    cc[0] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    cc[1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

// grid (slots * cpn, trees): stable partition of the chunk (wave w walks the
// chunk's quarter w in steps of 64 with ballot prefixes, starting from the
// counts of the node's earlier chunks and of the chunk's earlier quarters);
// the chunks of leaves are copied
__global__ __launch_bounds__(256) void wide_scatter(LevelArgs a) {
  __shared__ int wt[2][4];
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base;
  const int slot = blockIdx.x / a.wide_cpn, chunk = blockIdx.x % a.wide_cpn;
  int o, n, depth;
  wide_node(a, slot, &o, &n, &depth);
  const int32_t* pin = a.perm_in + (int64_t)tree * a.N;
  int32_t* pout = a.perm_out + (int64_t)tree * a.N;
  const uint64_t* hin = a.hpos_in + (int64_t)tree * a.N;
  uint64_t* hout = a.hpos_out + (int64_t)tree * a.N;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int i0 = chunk * kWideChunk, i1 = min(n, i0 + kWideChunk);
  if (depth < a.level || n <= a.c) {
    // leaf: copied once, by the slot whose remaining path bits are all zero
    const int below = a.level - depth;
    if (below > 0 && (slot & ((1 << below) - 1)) != 0) return;
    for (int i = i0 + tid; i < i1; i += 256) {
      pout[o + i] = pin[o + i];
      hout[o + i] = hin[o + i];
    }
    return;
  }
  if (i0 >= n) return;
  const int32_t* st = wide_state(a, tree, slot);
  const uint32_t kstar = (uint32_t)st[2];
  const int eq_take = st[3];   // members equal to kstar that go left (lowest positions)
  const int t = split_size(n, a.c);
  int lb = 0, eb = 0;   // members of the node's earlier chunks below / equal to kstar
  for (int q = 0; q < chunk; ++q) {
    const int32_t* cc = wide_counts(a, tree, slot, q);
    lb += cc[0];
    eb += cc[1];
  }
  const uint32_t* keys = a.keys + (int64_t)tree * a.N + o;
  const int per_w = kWideChunk / 4;
  const int r0 = min(i1, i0 + w * per_w), r1 = min(i1, r0 + per_w);
  int cl = 0, ce = 0;
  for (int i = r0 + l; i < r1; i += 64) {
    const uint32_t k = keys[i];
    cl += k < kstar;
    ce += k == kstar;
  }
  cl = wave_sum_int(cl);
  ce = wave_sum_int(ce);
  if (l == 0) { wt[0][w] = cl; wt[1][w] = ce; }
  __syncthreads();
  for (int q = 0; q < w; ++q) { lb += wt[0][q]; eb += wt[1][q]; }
  int erun = eb;                        // equal members before the current step
  int lrun = lb + min(eb, eq_take);     // left members before the current step
  constexpr int BATCH = 4;
  for (int base = r0; base < r1; base += 64 * BATCH) {
    uint32_t k[BATCH];
    int pv[BATCH];
    uint64_t hv[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + 64 * b + l;
      k[b] = 0u; pv[b] = 0; hv[b] = 0;
      if (i < r1) { k[b] = keys[i]; pv[b] = pin[o + i]; hv[b] = hin[o + i]; }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + 64 * b + l;
      const bool valid = i < r1;
      const bool less = valid && k[b] < kstar;
      const bool eq = valid && k[b] == kstar;
      uint64_t bal_e, bal_l;
      const int eqpre = lane_prefix(eq, &bal_e);
      const bool left = less || (eq && erun + eqpre < eq_take);
      const int lpre = lane_prefix(left, &bal_l);
      const int lrank = lrun + lpre;
      if (valid) {
        const int dest = left ? o + lrank : o + t + (i - lrank);
        if (dest < o + n) {   // holds by construction; guards the slice
          pout[dest] = pv[b];
          hout[dest] = hv[b];
        }
      }
      erun += __popcll(bal_e);
      lrun += __popcll(bal_l);
    }
  }
}

// Split of nodes of at most kSmallNode members: one wave per node (four per
// workgroup), the one-wave selection of wave_select.h; leaves are copied.
constexpr int kSmallNode = kWaveSelMax;

__global__ __launch_bounds__(256) void pddp_split_small(LevelArgs a) {
  __shared__ int hist[4][256];
  const int tree = (int)blockIdx.y * a.tree_step + a.tree_base, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int slot = blockIdx.x * 4 + w;
  if (slot >= (1 << a.level)) return;   // the whole wave
  int o = 0, m = a.N, depth = 0;
  for (; depth < a.level; ++depth) {
    if (m <= a.c) break;
    const int t = split_size(m, a.c);
    if ((slot >> (a.level - 1 - depth)) & 1) { o += t; m -= t; } else { m = t; }
  }
  const int32_t* pin = a.perm_in + (int64_t)tree * a.N;
  int32_t* pout = a.perm_out + (int64_t)tree * a.N;
  const uint64_t* hin = a.hpos_in + (int64_t)tree * a.N;
  uint64_t* hout = a.hpos_out + (int64_t)tree * a.N;
  if (depth < a.level || m <= a.c) {
    const int below = a.level - depth;
    if (below > 0 && (slot & ((1 << below) - 1)) != 0) return;
    for (int i = l; i < m; i += 64) {
      pout[o + i] = pin[o + i];
      hout[o + i] = hin[o + i];
    }
    return;
  }
  const int off = o, n = m;   // n <= kSmallNode (checked by the launch)
  const int t = split_size(n, a.c);
  const uint32_t* gkeys = a.keys + (int64_t)tree * a.N + off;
  wave_select(l, n, t, [&](int i) { return gkeys[i]; }, hist[w], [&](int i, bool left, int lrank) {
    const int dest = left ? off + lrank : off + t + (i - lrank);
    if (dest < off + n) {
      pout[dest] = pin[off + i];
      hout[dest] = hin[off + i];
    }
  });
}

// Largest node that splits at a level (host).
int max_split_node(int N, int c, int level) {
  struct R {
    static int rec(int n, int c, int l) {
      if (n <= c) return 0;
      if (l == 0) return n;
      const int t = split_size(n, c);
      const int x = rec(t, c, l - 1), y = rec(n - t, c, l - 1);
      return x > y ? x : y;
    }
  };
  return R::rec(N, c, level);
}

__global__ void perm_init(int32_t* perm, int trees, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)trees * N) perm[i] = (int32_t)(i % N);
}

__global__ void perm_out(const int32_t* perm_t, int tensor, int BH, int N, int kshare,
                         int32_t* perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)BH * N) return;
  const int64_t bh = i / N, p = i % N;
  if (tensor == 0) perm[i] = perm_t[(2 * bh) * N + p];
  else perm[i] = perm_t[(2 * (bh - bh % kshare) + 1) * N + p];   // the group's first head's key tree
}

// Means of the original rows of every cluster. Thread (row slot, group g)
// sums 16-byte groups of rows slot, slot + S, ... in order; the S partial sums
// of a group are then added in slot order.
template <typename T, int D>
__global__ __launch_bounds__(256) void centroids_kernel(const T* __restrict__ Q,
                                                        const T* __restrict__ K, int N, int c_q,
                                                        int c_k, const int32_t* __restrict__ pq,
                                                        const int32_t* __restrict__ pk,
                                                        float* __restrict__ cq,
                                                        float* __restrict__ ck,
                                                        int32_t* __restrict__ counts, int kvg,
                                                        int t0) {
  constexpr int EPG = 16 / (int)sizeof(T);   // elements per 16-byte group
  constexpr int NG = D / EPG;                // groups per row
  constexpr int S = 256 / NG;                // row slots
  __shared__ float part[S][D + 1];
  __shared__ int stoks[256];
  const int j = blockIdx.x, bh = blockIdx.y, tensor = (int)blockIdx.z + t0;
  const int c = tensor == 0 ? c_q : c_k;
  const int nc = (N + c - 1) / c;
  if (j >= nc) return;
  const int nj = min(c, N - j * c);
  const T* X = tensor == 0 ? Q + (int64_t)bh * N * D : K + (int64_t)(bh / kvg) * N * D;
  const int32_t* perm = (tensor == 0 ? pq : pk) + (int64_t)bh * N + (int64_t)j * c;
  const int tid = threadIdx.x;
  if (tid < nj) stoks[tid] = perm[tid];
  __syncthreads();
  const int g = tid % NG, slot = tid / NG;
  float acc[EPG];
#pragma unroll
  for (int e = 0; e < EPG; ++e) acc[e] = 0.0f;
#pragma unroll 4
  for (int r = slot; r < nj; r += S) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(X + (int64_t)stoks[r] * D + g * EPG);
    if constexpr (sizeof(T) == 2) {
      const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += bf16_to_f32((uint16_t)(ws[k] & 0xFFFFu));
        acc[2 * k + 1] += bf16_to_f32((uint16_t)(ws[k] >> 16));
      }
    } else {
      acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y);
      acc[2] += __uint_as_float(v.z); acc[3] += __uint_as_float(v.w);
    }
  }
#pragma unroll
  for (int e = 0; e < EPG; ++e) part[slot][g * EPG + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float sum = 0.0f;
    for (int q = 0; q < S; ++q) sum += part[q][tid];
    float* out = (tensor == 0 ? cq : ck) + ((int64_t)bh * nc + j) * D;
    out[tid] = sum / (float)nj;
    if (tid == 0 && tensor == 1 && counts) counts[(int64_t)bh * nc + j] = nj;   // key clusters
  }
}

}  // namespace

void launch_perm_init(int32_t* perm, int trees, int N, hipStream_t st) {
  const int64_t n = (int64_t)trees * N;
  perm_init<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, trees, N);
}

void launch_perm_out(const int32_t* perm_t, int tensor, int BH, int N, int kshare, int32_t* perm,
                     hipStream_t st) {
  const int64_t n = (int64_t)BH * N;
  perm_out<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm_t, tensor, BH, N, kshare, perm);
}

constexpr int64_t kDirSplitNodes = 2048;   // node slots of a level from which tensors launch apart

template <typename T, int D>
static void level_impl(const LevelArgs& a, hipStream_t st) {
  // the trees tree_base, tree_base + tree_step, ... below 2 BH
  const int trees = (2 * a.BH - a.tree_base + a.tree_step - 1) / a.tree_step;
  dim3 gslots(1u << a.level, trees);
  dim3 gspan((a.N + kSampleSpan - 1) / kSampleSpan, trees);
  // bf16 power-iteration levels whose nodes are small draw the sample inside
  // the direction kernel; the others take the per-chunk lists
  LevelArgs la = a;
  la.sample_inline = (sizeof(T) == 2 && a.split_mode == 0 &&
                      max_split_node(a.N, a.c, a.level) <= 32 * DirMma<D>::NT) ? 1 : 0;
  if (!la.sample_inline) pddp_sample<<<gspan, 256, 0, st>>>(la);
  if (a.split_mode == 1) {
    const int64_t nmax = ((int64_t)a.N >> a.level) + 2 * (int64_t)a.c;   // bounds every node
    const size_t lds = (size_t)((nmax + a.c - 1) / a.c + 2) * 4;
    pddp_dir_y<D><<<gslots, 256, lds, st>>>(a);
  } else if constexpr (sizeof(T) == 2) {
    const int64_t nmax = ((int64_t)a.N >> a.level) + 2 * (int64_t)a.c;   // bounds every node
    const size_t lds = (size_t)((nmax + a.c - 1) / a.c + 2) * 4;
    // levels with many nodes: one launch per tensor, so that the key trees
    // run at three workgroups per CU (the trees of a launch alternate between
    // query and key trees when its step is odd); levels with few nodes: one
    // launch (two would add a launch latency each)
    auto dir_launch = [&](const LevelArgs& l) {
      const int tr = (2 * a.BH - l.tree_base + l.tree_step - 1) / l.tree_step;
      if (tr <= 0) return;
      dim3 g(1u << a.level, tr);
      if ((l.tree_base & 1) == 0) pddp_dir_mma<D, 0><<<g, DirMma<D>::NT, lds, st>>>(l);
      else pddp_dir_mma<D, 1><<<g, DirMma<D>::NT, lds, st>>>(l);
    };
    // (counted over every tree of both tensors: the other trees' levels run
    // beside this launch on the other streams)
    const bool many = ((int64_t)2 * a.BH << a.level) >= kDirSplitNodes;
    if (!many) {
      pddp_dir_mma<D, -1><<<gslots, DirMma<D>::NT, lds, st>>>(la);
    } else if (la.tree_step % 2 == 0) {
      dir_launch(la);
    } else {
      LevelArgs l0 = la, l1 = la;
      l0.tree_step = l1.tree_step = 2 * la.tree_step;
      l1.tree_base = la.tree_base + la.tree_step;
      dir_launch(l0);
      dir_launch(l1);
    }
  } else {
    const size_t lds = dir_smem<T, D>(a.N, a.c, a.level);
    {   // raise the dynamic-LDS limit when a level needs more (host threads serialised)
      static std::mutex mu;
      static size_t lds_allowed = 0;
      std::lock_guard<std::mutex> lock(mu);
      if (lds > lds_allowed) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&pddp_dir<T, D>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        lds_allowed = lds;
      }
    }
    pddp_dir<T, D><<<gslots, 256, lds, st>>>(a);
  }
  dim3 gproj((a.N + a.c - 1) / a.c, trees);
  if (a.split_mode == 1) pddp_project_y<<<gproj, 256, 0, st>>>(a);
  else pddp_project<T, D><<<gproj, 256, 0, st>>>(a);
  const int maxn = max_split_node(a.N, a.c, a.level);
  if (a.wide && maxn >= kWideNode && (1 << a.level) <= kWideSlots) {
    // wide split: every node in chunks of kWideChunk positions
    LevelArgs lw = a;
    lw.wide_cpn = (maxn + kWideChunk - 1) / kWideChunk;
    dim3 gs(1u << a.level, trees), gc((1u << a.level) * lw.wide_cpn, trees);
    wide_init<<<gs, 256, 0, st>>>(lw, 0);
    wide_minmax<<<gc, 256, 0, st>>>(lw);
    wide_init<<<gs, 256, 0, st>>>(lw, 1);
    for (int r = 0; r < 4; ++r) {   // at most four 8-bit digits; finished nodes skip the rest
      wide_hist<<<gc, 256, 0, st>>>(lw);
      wide_pick<<<gs, 64, 0, st>>>(lw);
    }
    wide_count<<<gc, 256, 0, st>>>(lw);
    wide_scatter<<<gc, 256, 0, st>>>(lw);
    return;
  }
  if (maxn <= kSmallNode) {
    dim3 gsmall(((1u << a.level) + 3) / 4, trees);
    pddp_split_small<<<gsmall, 256, 0, st>>>(a);
  } else {
    // the level's largest node in LDS when it fits (the top levels have few,
    // large nodes: one workgroup per CU is enough there)
    LevelArgs ls = a;
    ls.split_cache = std::min(max_split_node(a.N, a.c, a.level), kSplitCacheMax);
    const size_t lds = (size_t)ls.split_cache * 4;
    if (a.level <= 1) {
      CA_MAX_LDS_ONCE(&pddp_split<kSplitThreadsTop>, (size_t)kSplitCacheMax * 4);
      pddp_split<kSplitThreadsTop><<<gslots, kSplitThreadsTop, lds, st>>>(ls);
    } else {
      CA_MAX_LDS_ONCE(&pddp_split<kSplitThreads>, (size_t)kSplitCacheMax * 4);
      pddp_split<kSplitThreads><<<gslots, kSplitThreads, lds, st>>>(ls);
    }
  }
}

// Workspace words of the wide split for trees of N tokens (0 if no level of
// such a tree goes wide).
size_t wide_split_words(int BH, int N, int c) {
  const int L = tree_levels_host(N, c);
  bool any = false;
  for (int l = 0; l < L && (1 << l) <= kWideSlots; ++l) any |= max_split_node(N, c, l) >= kWideNode;
  if (!any) return 0;
  const size_t cpn = ((size_t)N + kWideChunk - 1) / kWideChunk;
  return 2 * (size_t)BH * kWideSlots * (kWideState + 2 * cpn);
}

void launch_level(const LevelArgs& a, hipStream_t st) {
  if (a.dtype == 0) {
    if (a.D == 64) level_impl<uint16_t, 64>(a, st); else level_impl<uint16_t, 128>(a, st);
  } else {
    if (a.D == 64) level_impl<float, 64>(a, st); else level_impl<float, 128>(a, st);
  }
}

void launch_centroids(const void* Q, const void* K, int dtype, int BH, int N, int D, int c_q,
                      int c_k, const int32_t* pq, const int32_t* pk, float* cq, float* ck,
                      int32_t* counts, int kvg, int t0, int nt, hipStream_t st) {
  const int cmin = c_q < c_k ? c_q : c_k;
  dim3 g((N + cmin - 1) / cmin, BH, nt);
  if (dtype == 0) {
    const uint16_t* q = (const uint16_t*)Q;
    const uint16_t* k = (const uint16_t*)K;
    if (D == 64) centroids_kernel<uint16_t, 64><<<g, 256, 0, st>>>(q, k, N, c_q, c_k, pq, pk, cq, ck, counts, kvg, t0);
    else centroids_kernel<uint16_t, 128><<<g, 256, 0, st>>>(q, k, N, c_q, c_k, pq, pk, cq, ck, counts, kvg, t0);
  } else {
    const float* q = (const float*)Q;
    const float* k = (const float*)K;
    if (D == 64) centroids_kernel<float, 64><<<g, 256, 0, st>>>(q, k, N, c_q, c_k, pq, pk, cq, ck, counts, kvg, t0);
    else centroids_kernel<float, 128><<<g, 256, 0, st>>>(q, k, N, c_q, c_k, pq, pk, cq, ck, counts, kvg, t0);
  }
}

}  // namespace ca
