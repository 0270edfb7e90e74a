// Metric pass of the clustering (paper v1 §3.2.2, Eq. 12, 15 and 16):
//   M_q = Q^T Q / N,  kbar = mean(K),  M_k = K^T K / N - kbar kbar^T,
//   s_i = (q_i^T G q_i)^{-1/2} with G the query geometry (M_k or I),
// plus a 64-bit content hash of every token row of Q and K that decides the
// node subsamples. Second moments and q^T G q run on bf16 MFMA with fp32
// accumulation (G is split into three bf16 terms so q^T G q keeps fp32
// accuracy); fp32 inputs take a VALU path.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "mfma.h"

namespace ca {

namespace {

constexpr int kMetricTile = 128;  // tokens per LDS tile

// Row content hash: fmix64(sum_j w_j golden^(j+1) mod 2^64) over the row's
// 32-bit words; hash_word gives one term of the sum.
struct HashPow {
  uint64_t v[128];
};
constexpr HashPow make_hash_pow() {
  HashPow t{};
  uint64_t p = kGolden;
  for (int j = 0; j < 128; ++j) {
    t.v[j] = p;
    p *= kGolden;
  }
  return t;
}
__constant__ HashPow kHashPow = make_hash_pow();

CA_DEV uint64_t hash_word(uint32_t j, uint32_t w) { return (uint64_t)w * kHashPow.v[j]; }

// One workgroup per (chunk of rows, head, tensor): tiles of 128 tokens are
// read one round trip ahead as token pairs, stored transposed in LDS and fed
// to the matrix cores; the row hashes and the key sums come from the same
// registers.
template <int D>
__global__ __launch_bounds__(256) void metric_partial_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int N, int rows_per_chunk,
    int nchunks, float* __restrict__ partial, uint64_t* __restrict__ hash, int kvg) {
  constexpr int TT = kMetricTile;
  constexpr int NB = D / 32;
  constexpr int BPW = NB * NB / 4;          // 32x32 blocks per wave
  constexpr int LDT = TT + 8;               // padded token stride in LDS (272 B)
  constexpr int TP = TT / 2;                // token pairs per tile
  constexpr int GI = 256 / TP;              // group slots
  constexpr int GROUPS = D / 8;             // 16-byte groups per row
  constexpr int GPT = GROUPS / GI;          // groups per thread
  __shared__ __attribute__((aligned(16))) uint16_t sx[D][LDT];
  __shared__ uint64_t shash[GI][TT];

  const int bh = blockIdx.y, chunk = blockIdx.x, t = blockIdx.z;
  const int r0 = chunk * rows_per_chunk;
  const int r1 = min(N, r0 + rows_per_chunk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, r = l & 31;
  // thread (tp, gi): tokens 2 tp, 2 tp + 1 of each tile, groups gi + GI k
  const int tp = tid % TP, gi = tid / TP;
  const uint16_t* X = t == 0 ? Q + (int64_t)bh * N * D : K + (int64_t)(bh / kvg) * N * D;
  uint64_t hpow[GPT][4];
#pragma unroll
  for (int k = 0; k < GPT; ++k)
#pragma unroll
    for (int q = 0; q < 4; ++q) hpow[k][q] = kHashPow.v[4 * (gi + GI * k) + q];

  floatx16_t acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) acc[i] = zero16();
  float ksum[GPT][8];
#pragma unroll
  for (int k = 0; k < GPT; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) ksum[k][e] = 0.0f;

  u32x4_t pre[GPT][2];
  auto fetch = [&](int base) {
#pragma unroll
    for (int k = 0; k < GPT; ++k)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int tok = base + 2 * tp + q;
        pre[k][q] = u32x4_t{0u, 0u, 0u, 0u};
        if (tok < r1) pre[k][q] = *reinterpret_cast<const u32x4_t*>(X + (int64_t)tok * D + 8 * (gi + GI * k));
      }
  };
  fetch(r0);
  for (int base = r0; base < r1; base += TT) {
    uint64_t hp0 = 0, hp1 = 0;
#pragma unroll
    for (int k = 0; k < GPT; ++k) {
      const int g = gi + GI * k;
      const uint32_t a0[4] = {pre[k][0].x, pre[k][0].y, pre[k][0].z, pre[k][0].w};
      const uint32_t a1[4] = {pre[k][1].x, pre[k][1].y, pre[k][1].z, pre[k][1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hp0 += (uint64_t)a0[q] * hpow[k][q];
        hp1 += (uint64_t)a1[q] * hpow[k][q];
        // dims 8g + 2q (low halves) and 8g + 2q + 1 (high halves) of the two tokens
        *reinterpret_cast<uint32_t*>(&sx[8 * g + 2 * q][2 * tp]) = (a0[q] & 0xFFFFu) | (a1[q] << 16);
        *reinterpret_cast<uint32_t*>(&sx[8 * g + 2 * q + 1][2 * tp]) = (a0[q] >> 16) | (a1[q] & 0xFFFF0000u);
        if (t == 1) {
          ksum[k][2 * q] += bf16_to_f32((uint16_t)(a0[q] & 0xFFFFu)) + bf16_to_f32((uint16_t)(a1[q] & 0xFFFFu));
          ksum[k][2 * q + 1] += bf16_to_f32((uint16_t)(a0[q] >> 16)) + bf16_to_f32((uint16_t)(a1[q] >> 16));
        }
      }
    }
    shash[gi][2 * tp] = hp0;
    shash[gi][2 * tp + 1] = hp1;
    __syncthreads();
    if (base + TT < r1) fetch(base + TT);   // next tile in flight during the products
    if (tid < TT && base + tid < r1) {
      uint64_t s = 0;
#pragma unroll
      for (int q = 0; q < GI; ++q) s += shash[q][tid];
      hash[((int64_t)bh * 2 + t) * N + base + tid] = fmix64(s);
    }
#pragma unroll
    for (int s = 0; s < TT / 16; ++s) {
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int b = w * BPW + i, bm = b / NB, bn = b % NB;
        bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sx[bm * 32 + r][s * 16 + h * 8]);
        bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&sx[bn * 32 + r][s * 16 + h * 8]);
        acc[i] = mfma32(a, bb, acc[i]);
      }
    }
    __syncthreads();
  }

  float* out = partial + ((int64_t)bh * nchunks + chunk) * (2 * D * D + D);
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = w * BPW + i, bm = b / NB, bn = b % NB;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      out[t * D * D + (bm * 32 + c_row(e, h)) * D + bn * 32 + r] = acc[i][e];
  }
  if (t == 1) {
    // key sums: the TP token-pair lanes of a group (fixed butterfly order)
#pragma unroll
    for (int k = 0; k < GPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = ksum[k][e];
#pragma unroll
        for (int o = 1; o < TP; o <<= 1) v += __shfl_xor(v, o, 64);
        if (tp == 0) out[2 * D * D + 8 * (gi + GI * k) + e] = v;
      }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void metric_partial_f32(
    const T* __restrict__ Q, const T* __restrict__ K, int N, int rows_per_chunk, int nchunks,
    float* __restrict__ partial, uint64_t* __restrict__ hash, int kvg) {
  // Plain VALU path: thread e accumulates entries e, e+256, ... of Q^T Q and K^T K.
  constexpr int TT = 32;
  __shared__ float sx[2][TT][D];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int r0 = chunk * rows_per_chunk;
  const int r1 = min(N, r0 + rows_per_chunk);
  const int tid = threadIdx.x;
  const T* X[2] = {Q + (int64_t)bh * N * D, K + (int64_t)(bh / kvg) * N * D};
  constexpr int PER = (D * D + 255) / 256;
  float aq[PER], ak[PER];
  for (int i = 0; i < PER; ++i) aq[i] = ak[i] = 0.0f;
  float ks = 0.0f;
  for (int base = r0; base < r1; base += TT) {
    for (int e = tid; e < 2 * TT * D; e += 256) {
      const int t = e / (TT * D), rr = (e / D) % TT, dd = e % D;
      sx[t][rr][dd] = (base + rr < r1) ? load_elem(X[t], (int64_t)(base + rr) * D + dd) : 0.0f;
    }
    __syncthreads();
    if (tid < 2 * TT) {
      const int t = tid / TT, rr = tid % TT;
      if (base + rr < r1) {
        uint64_t s = 0;
        const T* row = X[t] + (int64_t)(base + rr) * D;
        const uint32_t* wrow = reinterpret_cast<const uint32_t*>(row);
        constexpr int W = D * (int)sizeof(T) / 4;
        for (int j = 0; j < W; ++j) s += hash_word((uint32_t)j, wrow[j]);
        hash[((int64_t)bh * 2 + t) * N + base + rr] = fmix64(s);
      }
    }
    for (int rr = 0; rr < TT; ++rr) {
      for (int i = 0; i < PER; ++i) {
        const int e = tid + 256 * i;
        if (e < D * D) {
          const int a = e / D, b = e % D;
          aq[i] += sx[0][rr][a] * sx[0][rr][b];
          ak[i] += sx[1][rr][a] * sx[1][rr][b];
        }
      }
      if (tid < D) ks += sx[1][rr][tid];
    }
    __syncthreads();
  }
  float* out = partial + ((int64_t)bh * nchunks + chunk) * (2 * D * D + D);
  for (int i = 0; i < PER; ++i) {
    const int e = tid + 256 * i;
    if (e < D * D) {
      out[e] = aq[i];
      out[D * D + e] = ak[i];
    }
  }
  if (tid < D) out[2 * D * D + tid] = ks;
}

// Sum the chunk partials in chunk order; write M_q, M_k (fp32), kbar and the
// three-term bf16 split of the query geometry G (M_k, or I without transform).
template <int D>
__global__ __launch_bounds__(256) void metric_reduce(const float* __restrict__ partial,
                                                     int nchunks, int N, int transform,
                                                     float* __restrict__ Mq,
                                                     float* __restrict__ Mk,
                                                     float* __restrict__ kbar,
                                                     uint16_t* __restrict__ gsplit,
                                                     float* __restrict__ Mpk) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const int a = e / D, b = e % D;
  const float* p = partial + (int64_t)bh * nchunks * (2 * D * D + D);
  float sq = 0.0f, sk = 0.0f, ka = 0.0f, kb = 0.0f;
  for (int ch = 0; ch < nchunks; ++ch) {
    const float* pc = p + (int64_t)ch * (2 * D * D + D);
    sq += pc[e];
    sk += pc[D * D + e];
    ka += pc[2 * D * D + a];
    kb += pc[2 * D * D + b];
  }
  const float invN = 1.0f / (float)N;
  const float mq = sq * invN;
  const float kma = ka * invN, kmb = kb * invN;
  const float mk = sk * invN - kma * kmb;
  Mq[(int64_t)bh * D * D + e] = mq;
  Mk[(int64_t)bh * D * D + e] = mk;
  {
    // element (a, b) sits in wave b/32, lane (b % 32) + 32 h, slot 16 (a/32) + i of
    // the direction kernel, where a % 32 = 8 (i/4) + 4 h + i % 4 (the MFMA
    // accumulator row order)
    const int rr = a & 31, hh = (rr >> 2) & 1, ii = 4 * (rr >> 3) + (rr & 3);
    const int64_t pk = (int64_t)((b >> 5) * 64 + (b & 31) + 32 * hh) * (D / 2) + 16 * (a >> 5) + ii;
    Mpk[(int64_t)(2 * bh) * D * D + pk] = mk;
    Mpk[(int64_t)(2 * bh + 1) * D * D + pk] = mq;
  }
  if (a == 0) kbar[(int64_t)bh * D + b] = kmb;
  const float g = transform ? mk : (a == b ? 1.0f : 0.0f);
  const uint16_t hi = f32_to_bf16(g);
  const float r1 = g - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r1);
  const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
  uint16_t* gs = gsplit + (int64_t)bh * 3 * D * D;
  gs[e] = hi;
  gs[D * D + e] = mid;
  gs[2 * D * D + e] = lo;
}

// queries per workgroup of qnorm_bf16: the fewest that keep every workgroup
// resident at once (three per CU at its register count), whole 32-query tiles
int qnorm_span(int N, int BH) {
  const int per_head = std::max(1, 768 / BH);
  const int span = (N + per_head - 1) / per_head;
  return (span + 31) / 32 * 32;
}

// Upper block triangle of the symmetric query geometry G, in 16-wide k-steps
// of 32-row blocks: q^T G q = sum_I q_I^T (G_II q_I + sum_{J > I} 2 G_IJ q_J),
// so block row I covers k-steps [2 I, D / 16), and the blocks right of the
// diagonal enter doubled (exact in bf16). The k-steps are dealt to the waves
// of a query group in at most two segments (block row, first, end) each, the
// same number of k-steps per wave: at D = 128, 20 k-steps over 4 waves
// (10 of the 16 blocks), at D = 64, 6 over 2 waves.
struct QnSeg {
  int row, s0, s1;
};
template <int D>
struct QnPlan;
template <>
struct QnPlan<128> {
  static constexpr int KMAX = 5;
  static constexpr QnSeg seg[4][2] = {{{0, 0, 5}, {0, 0, 0}},
                                      {{0, 5, 8}, {3, 6, 8}},
                                      {{1, 2, 7}, {1, 0, 0}},
                                      {{1, 7, 8}, {2, 4, 8}}};
};
template <>
struct QnPlan<64> {
  static constexpr int KMAX = 3;
  static constexpr QnSeg seg[2][2] = {{{0, 0, 3}, {0, 0, 0}}, {{0, 3, 4}, {1, 2, 4}}};
};

CA_DEV bf16x8_t bf16x8_times2(const bf16x8_t& v) {
  const u32x4_t u = __builtin_bit_cast(u32x4_t, v);
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = f32_to_bf16(2.0f * bf16_to_f32((uint16_t)(u[k] & 0xFFFFu)));
    const uint32_t hi = f32_to_bf16(2.0f * bf16_to_f32((uint16_t)(u[k] >> 16)));
    o[k] = lo | (hi << 16);
  }
  return as_bf16x8(o);
}

// s_i = (q_i^T G q_i)^{-1/2} (0 if q^T G q <= 0). The products run on the
// matrix cores with G as hi + mid + lo bf16 terms held as A operands for the
// block's lifetime (the wave's k-steps of the upper block triangle, see
// QnPlan); query tiles stream through LDS (double-buffered) as B operands,
// then each wave dots its accumulator rows with the query and the waves'
// partial sums are added in wave order.
template <int D>
__global__ __launch_bounds__(256) void qnorm_bf16(const uint16_t* __restrict__ Q, int N, int span,
                                                  const uint16_t* __restrict__ gsplit,
                                                  float* __restrict__ s_out) {
  constexpr int NB = D / 32;                 // waves per query group
  constexpr int QG = 4 / NB;                 // query groups of 32 per tile
  constexpr int KMAX = QnPlan<D>::KMAX;
  constexpr int QP = D + 8;                  // padded query row (bf16)
  constexpr int TILE = 32 * QG;              // queries per step
  constexpr int PPT = TILE * D / 8 / 256;    // 16-byte pieces per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][TILE][QP];
  __shared__ float tred[2][NB][TILE];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, h = l >> 5, r = l & 31;
  const int bn = w % NB, qg = w / NB;
  const uint16_t* Qh = Q + (int64_t)bh * N * D;
  const uint16_t* G = gsplit + (int64_t)bh * 3 * D * D;
  const int q0 = blockIdx.x * span;
  const int qend = min(N, q0 + span);

  // register staging of two tiles: tile t + 1 is stored to LDS while tile t
  // is in the matrix cores, and tile t + 3 is requested in its place
  u32x4_t st[2][PPT];
  auto load_tile = [&](u32x4_t (&dst)[PPT], int t0) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int idx = tid + 256 * k, row = idx / (D / 8), pc = idx % (D / 8);
      dst[k] = u32x4_t{0u, 0u, 0u, 0u};
      if (t0 + row < qend) dst[k] = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)(t0 + row) * D + 8 * pc);
    }
  };
  auto store_tile = [&](const u32x4_t (&src)[PPT], int buf) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int idx = tid + 256 * k, row = idx / (D / 8), pc = idx % (D / 8);
      *reinterpret_cast<u32x4_t*>(&sq[buf][row][8 * pc]) = src[k];
    }
  };
  load_tile(st[0], q0);
  if (q0 + TILE < qend) load_tile(st[1], q0 + TILE);
  // A operands of the wave's k-steps, in segment order: rows [32 row, +32)
  // of the three parts of G, doubled right of the diagonal block
  const QnSeg sg0 = QnPlan<D>::seg[bn][0], sg1 = QnPlan<D>::seg[bn][1];
  const int n0 = sg0.s1 - sg0.s0, n1 = sg1.s1 - sg1.s0;
  bf16x8_t ga[3][KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const bool first = k < n0;
    const int row = first ? sg0.row : sg1.row;
    const int sk = first ? sg0.s0 + k : sg1.s0 + (k - n0);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(G + (int64_t)p * D * D +
                                                      (int64_t)(32 * row + r) * D + 16 * sk + 8 * h);
      if ((sk >> 1) > row) v = bf16x8_times2(v);
      ga[p][k] = v;
    }
  }
  store_tile(st[0], 0);
  if (q0 + 2 * TILE < qend) load_tile(st[0], q0 + 2 * TILE);
  __syncthreads();
  // one tile: the wave's segments on the matrix cores, its partial
  // sum_I q_I^T y_I, then the next tile's store
  auto step = [&](int t0, auto parity) __attribute__((always_inline)) {
    constexpr int buf = decltype(parity)::value;
    const uint16_t* qrow = &sq[buf][32 * qg + r][0];
    // lane (r, h) holds y[32 row + c_row(i, h)][query r] of a segment
    auto dot = [&](const floatx16_t& y, int row, float tp) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x2_t qv = *reinterpret_cast<const u32x2_t*>(qrow + 32 * row + 8 * jq + 4 * h);
        tp = fmaf(y[4 * jq + 0], bf16_to_f32((uint16_t)(qv.x & 0xFFFFu)), tp);
        tp = fmaf(y[4 * jq + 1], bf16_to_f32((uint16_t)(qv.x >> 16)), tp);
        tp = fmaf(y[4 * jq + 2], bf16_to_f32((uint16_t)(qv.y & 0xFFFFu)), tp);
        tp = fmaf(y[4 * jq + 3], bf16_to_f32((uint16_t)(qv.y >> 16)), tp);
      }
      return tp;
    };
    // the segments one after the other through one accumulator
    float tp = 0.0f;
    floatx16_t y = zero16();
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k == n0) {   // the first segment is complete
        tp = dot(y, sg0.row, tp);
        y = zero16();
      }
      const int sk = k < n0 ? sg0.s0 + k : sg1.s0 + (k - n0);
      const bf16x8_t bq = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * sk + 8 * h);
#pragma unroll
      for (int p = 0; p < 3; ++p) y = mfma32(ga[p][k], bq, y);
    }
    tp = dot(y, n1 > 0 ? sg1.row : sg0.row, tp);
    tp = sum_halves(tp);
    if (h == 0) tred[buf][bn][32 * qg + r] = tp;
    // tile t + 1 (staged in slot buf ^ 1) into the other LDS buffer, and
    // tile t + 3 requested into that slot
    if (t0 + TILE < qend) {
      store_tile(st[buf ^ 1], buf ^ 1);
      if (t0 + 3 * TILE < qend) load_tile(st[buf ^ 1], t0 + 3 * TILE);
    }
    __syncthreads();
    if (tid < TILE && t0 + tid < qend) {
      float t = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) t += tred[buf][b][tid];
      s_out[(int64_t)bh * N + t0 + tid] = t > 0.0f ? 1.0f / sqrtf(t) : 0.0f;
    }
  };
  for (int t0 = q0; t0 < qend; t0 += 2 * TILE) {
    step(t0, std::integral_constant<int, 0>{});
    if (t0 + TILE < qend) step(t0 + TILE, std::integral_constant<int, 1>{});
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void qnorm_f32(const T* __restrict__ Q, int N,
                                                 const float* __restrict__ Mk, int transform,
                                                 float* __restrict__ s_out) {
  __shared__ float G[D][D];
  const int bh = blockIdx.y;
  for (int e = threadIdx.x; e < D * D; e += 256)
    G[e / D][e % D] = transform ? Mk[(int64_t)bh * D * D + e] : ((e / D) == (e % D) ? 1.0f : 0.0f);
  __syncthreads();
  const int tok = blockIdx.x * 256 + threadIdx.x;
  if (tok >= N) return;
  const T* q = Q + ((int64_t)bh * N + tok) * D;
  float qv[D];
  for (int j = 0; j < D; ++j) qv[j] = load_elem(q, j);
  float t = 0.0f;
  for (int j = 0; j < D; ++j) {
    float y = 0.0f;
    for (int k = 0; k < D; ++k) y += G[j][k] * qv[k];
    t += qv[j] * y;
  }
  s_out[(int64_t)bh * N + tok] = t > 0.0f ? 1.0f / sqrtf(t) : 0.0f;
}

__global__ void fill_f32(float* p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

int metric_rows_per_chunk(int N, int BH) {
  // as many chunks as keep every workgroup of the pass resident at once (two
  // per CU at the bf16 kernel's register count: 512 workgroups with the two
  // tensors), at least 256 rows each, a multiple of the 128-token tile
  const int64_t want = std::max<int64_t>(1, 256 / BH);
  const int64_t most = ((int64_t)N + 255) / 256;
  const int64_t chunks = want < most ? want : most;
  const int64_t rows = ((int64_t)N + chunks - 1) / chunks;
  return (int)((rows + kMetricTile - 1) / kMetricTile * kMetricTile);
}

// Mean of the query metrics of each group of g heads, into the slots of the
// group's first head (in place: every thread reads all of its element's
// inputs before writing). Mpk's packing is an element permutation, so the
// packed copy is averaged the same way.
__global__ __launch_bounds__(256) void pool_key_metric(float* __restrict__ Mq, float* __restrict__ Mpk,
                                                       int DD, int g) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lead = blockIdx.y * g;
  if (e >= DD) return;
  float a = 0.0f, b = 0.0f;
  for (int i = 0; i < g; ++i) {
    a += Mq[(int64_t)(lead + i) * DD + e];
    b += Mpk[(int64_t)(2 * (lead + i) + 1) * DD + e];
  }
  Mq[(int64_t)lead * DD + e] = a / (float)g;
  Mpk[(int64_t)(2 * lead + 1) * DD + e] = b / (float)g;
}

void launch_pool_key_metric(float* Mq, float* Mpk, int BH, int D, int g, hipStream_t st) {
  dim3 grid((D * D + 255) / 256, BH / g);
  pool_key_metric<<<grid, 256, 0, st>>>(Mq, Mpk, D * D, g);
}

void launch_metric(const void* Q, const void* K, int dtype, int BH, int N, int D, int transform,
                   float* partial, uint64_t* hash, float* Mq, float* Mk, float* kbar,
                   uint16_t* gsplit, float* Mpk, int kvg, hipStream_t st) {
  const int rows = metric_rows_per_chunk(N, BH);
  const int nchunks = (N + rows - 1) / rows;
  dim3 gp(nchunks, BH);
  if (dtype == 0) {
    const uint16_t* q = (const uint16_t*)Q;
    const uint16_t* k = (const uint16_t*)K;
    gp.z = 2;
    if (D == 64) metric_partial_bf16<64><<<gp, 256, 0, st>>>(q, k, N, rows, nchunks, partial, hash, kvg);
    else metric_partial_bf16<128><<<gp, 256, 0, st>>>(q, k, N, rows, nchunks, partial, hash, kvg);
  } else {
    const float* q = (const float*)Q;
    const float* k = (const float*)K;
    if (D == 64) metric_partial_f32<float, 64><<<gp, 256, 0, st>>>(q, k, N, rows, nchunks, partial, hash, kvg);
    else metric_partial_f32<float, 128><<<gp, 256, 0, st>>>(q, k, N, rows, nchunks, partial, hash, kvg);
  }
  dim3 gr((D * D + 255) / 256, BH);
  if (D == 64) metric_reduce<64><<<gr, 256, 0, st>>>(partial, nchunks, N, transform, Mq, Mk, kbar, gsplit, Mpk);
  else metric_reduce<128><<<gr, 256, 0, st>>>(partial, nchunks, N, transform, Mq, Mk, kbar, gsplit, Mpk);
}

void launch_qnorm(const void* Q, int dtype, int BH, int N, int D, int transform,
                  int query_normalize, const uint16_t* gsplit, const float* Mk, float* s,
                  hipStream_t st) {
  if (!query_normalize) {
    int64_t n = (int64_t)BH * N;
    fill_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(s, n, 1.0f);
    return;
  }
  if (dtype == 0) {
    const int span = qnorm_span(N, BH);
    dim3 gq((N + span - 1) / span, BH);
    if (D == 64) qnorm_bf16<64><<<gq, 256, 0, st>>>((const uint16_t*)Q, N, span, gsplit, s);
    else qnorm_bf16<128><<<gq, 256, 0, st>>>((const uint16_t*)Q, N, span, gsplit, s);
  } else {
    dim3 gq((N + 255) / 256, BH);
    if (D == 64) qnorm_f32<float, 64><<<gq, 256, 0, st>>>((const float*)Q, N, Mk, transform, s);
    else qnorm_f32<float, 128><<<gq, 256, 0, st>>>((const float*)Q, N, Mk, transform, s);
  }
}

}  // namespace ca
