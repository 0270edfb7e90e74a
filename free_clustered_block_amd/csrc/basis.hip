// Principal-component basis for diagonalized recursive splitting (paper v1
// §3.2.1 "Diagonalized recursive splitting"; later revision §4.1.1): the
// vectors of each tree are rotated once into the principal-component basis of
// the whole set, taken in the transform's geometry (the metric M of v1 §3.2.2:
// z = F^T x for any factor F F^T = M), and every node then splits along the
// coordinate of highest sample variance.
//
//   qmoment_partial / qmoment_reduce   C_q = Cov(s q) over all queries (the
//       query representation x = s q of Eq. 16); the key covariance is M_k of
//       the metric pass.
//   basis_kernel   one workgroup per tree: pivoted Cholesky factor F of the
//       geometry M, Z = F^T C_x F, eigendecomposition of Z (-> W, lam), a_j = F w_j by
//       descending eigenvalue, each signed so that its largest-magnitude entry
//       is positive; writes A^T, so row j of the output is the direction whose
//       projection x . a_j is coordinate j.
//   basis_split / rotate_*   Y = the coordinates of every vector, once.
#include "kernels.h"
#include "mfma.h"

namespace ca {

namespace {

constexpr int kMomTile = 64;   // tokens per LDS tile of the bf16 moment pass

// Weighted second moment sum_t w_t q_t q_t^T (w = s^2) and sum_t s_t q_t over
// a chunk of query rows, on bf16 MFMA: the A operand is q (exact in bf16), the
// B operand w q split into three bf16 terms (fp32 accuracy). Thread (tp, gi)
// reads 16-byte groups of dims of the token pair (2 tp, 2 tp + 1) and writes
// them transposed as 32-bit words (the two tokens of one dim), the next tile
// in flight during the products.
template <int D>
__global__ __launch_bounds__(256) void qmoment_partial_bf16(const uint16_t* __restrict__ Q,
                                                            const float* __restrict__ s, int N,
                                                            int rows_per_chunk, int nchunks,
                                                            float* __restrict__ partial) {
  constexpr int TT = kMomTile;
  constexpr int NB = D / 32;
  constexpr int BPW = NB * NB / 4;          // 32x32 blocks per wave
  constexpr int LDT = TT + 8;
  constexpr int TP = TT / 2, GI = 256 / TP, GROUPS = D / 8, GPT = GROUPS / GI;
  __shared__ __attribute__((aligned(16))) uint16_t sx[D][LDT];
  __shared__ __attribute__((aligned(16))) uint16_t sw3[3][D][LDT];
  __shared__ float sv[2][TT];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int r0 = chunk * rows_per_chunk, r1 = min(N, r0 + rows_per_chunk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, r = l & 31;
  const int tp = tid % TP, gi = tid / TP;
  const uint16_t* X = Q + (int64_t)bh * N * D;
  const float* sq = s + (int64_t)bh * N;
  floatx16_t acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) acc[i] = zero16();
  float s1 = 0.0f;   // sum of s q over dim tid (tid < D), in token order
  u32x4_t pre[GPT][2];
  float ps[2];
  auto fetch = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tok = base + 2 * tp + q;
      ps[q] = tok < r1 ? sq[tok] : 0.0f;
#pragma unroll
      for (int k = 0; k < GPT; ++k) {
        pre[k][q] = u32x4_t{0u, 0u, 0u, 0u};
        if (tok < r1) pre[k][q] = *reinterpret_cast<const u32x4_t*>(X + (int64_t)tok * D + 8 * (gi + GI * k));
      }
    }
  };
  fetch(r0);
  int buf = 0;
  for (int base = r0; base < r1; base += TT) {
    const float w0 = ps[0] * ps[0], w1 = ps[1] * ps[1];
    if (gi == 0) {
      sv[buf][2 * tp] = ps[0];
      sv[buf][2 * tp + 1] = ps[1];
    }
#pragma unroll
    for (int k = 0; k < GPT; ++k) {
      const int g = gi + GI * k;
      const uint32_t a0[4] = {pre[k][0].x, pre[k][0].y, pre[k][0].z, pre[k][0].w};
      const uint32_t a1[4] = {pre[k][1].x, pre[k][1].y, pre[k][1].z, pre[k][1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {   // dim 8 g + 2 q + u
          const uint32_t b0 = (a0[q] >> (16 * u)) & 0xFFFFu, b1 = (a1[q] >> (16 * u)) & 0xFFFFu;
          const int dd = 8 * g + 2 * q + u;
          *reinterpret_cast<uint32_t*>(&sx[dd][2 * tp]) = b0 | (b1 << 16);
          const float x0 = bf16_to_f32((uint16_t)b0) * w0, x1 = bf16_to_f32((uint16_t)b1) * w1;
          const uint16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
          const float e0 = x0 - bf16_to_f32(h0), e1 = x1 - bf16_to_f32(h1);
          const uint16_t m0 = f32_to_bf16(e0), m1 = f32_to_bf16(e1);
          const uint16_t l0 = f32_to_bf16(e0 - bf16_to_f32(m0)), l1 = f32_to_bf16(e1 - bf16_to_f32(m1));
          *reinterpret_cast<uint32_t*>(&sw3[0][dd][2 * tp]) = (uint32_t)h0 | ((uint32_t)h1 << 16);
          *reinterpret_cast<uint32_t*>(&sw3[1][dd][2 * tp]) = (uint32_t)m0 | ((uint32_t)m1 << 16);
          *reinterpret_cast<uint32_t*>(&sw3[2][dd][2 * tp]) = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
      }
    }
    __syncthreads();
    if (base + TT < r1) fetch(base + TT);   // next tile in flight during the products
    if (tid < D) {
      const int nt = min(TT, r1 - base);
      for (int t = 0; t < nt; ++t) s1 = fmaf(sv[buf][t], bf16_to_f32(sx[tid][t]), s1);
    }
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      const int k0 = 16 * ks + 8 * h;
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int b = w * BPW + i, bm = b / NB, bn = b % NB;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sx[bm * 32 + r][k0]);
#pragma unroll
        for (int t = 0; t < 3; ++t)
          acc[i] = mfma32(a, *reinterpret_cast<const bf16x8_t*>(&sw3[t][bn * 32 + r][k0]), acc[i]);
      }
    }
    __syncthreads();
    buf ^= 1;
  }
  float* out = partial + ((int64_t)bh * nchunks + chunk) * (D * D + D);
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = w * BPW + i, bm = b / NB, bn = b % NB;
#pragma unroll
    for (int e = 0; e < 16; ++e) out[(bm * 32 + c_row(e, h)) * D + bn * 32 + r] = acc[i][e];
  }
  if (tid < D) out[D * D + tid] = s1;
}

// The same moments on fp32 rows, on the VALU: thread e accumulates entries
// e, e + 256, ... of the matrix over the chunk's tokens in order.
template <int D>
__global__ __launch_bounds__(256) void qmoment_partial_f32(const float* __restrict__ Q,
                                                           const float* __restrict__ s, int N,
                                                           int rows_per_chunk, int nchunks,
                                                           float* __restrict__ partial) {
  constexpr int TT = 32;
  __shared__ float sx[TT][D];
  __shared__ float sv[TT];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int r0 = chunk * rows_per_chunk, r1 = min(N, r0 + rows_per_chunk);
  const int tid = threadIdx.x;
  const float* X = Q + (int64_t)bh * N * D;
  const float* sq = s + (int64_t)bh * N;
  constexpr int EPT = (D * D + 255) / 256;
  float acc[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) acc[k] = 0.0f;
  float s1 = 0.0f;
  for (int base = r0; base < r1; base += TT) {
    const int nt = min(TT, r1 - base);
    for (int e = tid; e < TT * D; e += 256) {
      const int t = e / D, d = e % D;
      sx[t][d] = t < nt ? X[(int64_t)(base + t) * D + d] : 0.0f;
    }
    if (tid < TT) sv[tid] = tid < nt ? sq[base + tid] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + 256 * k;
      if (e < D * D) {
        const int a = e / D, b = e % D;
        for (int t = 0; t < nt; ++t) acc[k] = fmaf(sv[t] * sv[t] * sx[t][a], sx[t][b], acc[k]);
      }
    }
    if (tid < D)
      for (int t = 0; t < nt; ++t) s1 = fmaf(sv[t], sx[t][tid], s1);
    __syncthreads();
  }
  float* out = partial + ((int64_t)bh * nchunks + chunk) * (D * D + D);
#pragma unroll
  for (int k = 0; k < EPT; ++k)
    if (tid + 256 * k < D * D) out[tid + 256 * k] = acc[k];
  if (tid < D) out[D * D + tid] = s1;
}

// C_q = S2 / N - m m^T with m = S1 / N, chunk partials summed in chunk order.
template <int D>
__global__ __launch_bounds__(256) void qmoment_reduce(const float* __restrict__ partial, int nchunks,
                                                      int N, float* __restrict__ Cq) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const int a = e / D, b = e % D;
  const float* p = partial + (int64_t)bh * nchunks * (D * D + D);
  float s2 = 0.0f, ma = 0.0f, mb = 0.0f;
  for (int ch = 0; ch < nchunks; ++ch) {
    const float* pc = p + (int64_t)ch * (D * D + D);
    s2 += pc[e];
    ma += pc[D * D + a];
    mb += pc[D * D + b];
  }
  const float invN = 1.0f / (float)N;
  Cq[(int64_t)bh * D * D + e] = s2 * invN - (ma * invN) * (mb * invN);
}

// ----------------------------------------------------------------------------
// Symmetric eigendecomposition of a D x D matrix by one workgroup of 256
// threads (the textbook pipeline: Householder tridiagonalization, bisection on
// Sturm counts, inverse iteration, modified Gram-Schmidt, back-transform).
//
//   tridiagonalize  the matrix lives in registers, TPR = 256/D threads per row
//                   (EPT contiguous columns each); for k = 0 .. D-3 the
//                   reflector H_k = I - beta_k v_k v_k^T zeroes column k below
//                   the subdiagonal of the trailing block; v_k goes to row k of
//                   Hv (LDS, zero outside (k, D)); three barriers per step;
//   bisection       PPE = 256/D lanes per eigenvalue evaluate Sturm counts at
//                   PPE interior points, so each round shrinks the bracket by
//                   PPE + 1, down to 2^-22 of the Gershgorin bound;
//   inverse iter.   one lane per eigenvalue: three solves (T - lam I) x = b with
//                   the LDL^T factors formed on the fly (pivots below
//                   2^-23 |T| raised to it), L in registers, x in LDS;
//   MGS             two passes in descending eigenvalue order, each vector
//                   normalised, then removed from every vector after it;
//   back-transform  x <- H_0 ... H_{D-3} x.
//
// Eigenvalues ascend in lam; row j of Xv (global, D x D) is the unit
// eigenvector of lam[j].
// ----------------------------------------------------------------------------

template <int D>
struct EigLds {
  static constexpr int P = D + 1;
  float* S;      // in: [D][P] (destroyed); then Hv [D][D]
  float* Zw;     // [D][D]: inverse-iteration vectors, Zw[i D + j] = x_j[i]
  float* d;      // [D] diagonal of T
  float* e;      // [D] e[k] = T[k+1][k]
  float* e2;     // [D] e^2
  float* beta;   // [D]
  float* pb;     // [2][D] p of the current reflector (by step parity)
  float* red;    // [2][4]
  float* xb;     // [2][D] vectors broadcast during MGS
};

CA_DEV float ii_start(int i, int j) {
  uint32_t h = (uint32_t)(i + 1) * 0x9E3779B1u ^ (uint32_t)(j + 1) * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return (float)(h >> 8) * 0x1p-24f - 0.5f;
}

CA_DEV float rcpf(float x) { return __builtin_amdgcn_rcpf(x); }

// Wave reductions on DPP moves (VALU, no LDS round trip): lanes without a
// source read the identity. Row shifts build each 16-lane row's prefix, the
// two row broadcasts carry it across rows, lane 63 ends with the total.
template <int CTRL, int ROW_MASK>
CA_DEV float dpp_or(float x, float ident) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xf, false));
}
CA_DEV float wave_sum_dpp(float v) {
  v += dpp_or<0x111, 0xf>(v, 0.0f);   // row_shr:1
  v += dpp_or<0x112, 0xf>(v, 0.0f);   // row_shr:2
  v += dpp_or<0x114, 0xf>(v, 0.0f);   // row_shr:4
  v += dpp_or<0x118, 0xf>(v, 0.0f);   // row_shr:8
  v += dpp_or<0x142, 0xa>(v, 0.0f);   // row_bcast:15 into rows 1, 3
  v += dpp_or<0x143, 0xc>(v, 0.0f);   // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
CA_DEV float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_or<0x111, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_or<0x112, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_or<0x114, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_or<0x118, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_or<0x142, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_or<0x143, 0xc>(v, -INFINITY));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// sum over aligned groups of G = 2 or 4 adjacent lanes (quad permutations)
template <int G>
CA_DEV float group_sum(float v) {
  v += dpp_or<0xB1, 0xf>(v, 0.0f);                  // lane ^ 1
  if constexpr (G == 4) v += dpp_or<0x4E, 0xf>(v, 0.0f);   // lane ^ 2
  return v;
}

template <int D>
CA_DEV void eig_sym(const EigLds<D>& E, float* lam, float* __restrict__ Xv) {
  constexpr int P = EigLds<D>::P, TPR = 256 / D, EPT = D / TPR;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;

  // --- Householder tridiagonalization, rows in registers --------------------
  {
    const int r = tid / TPR, cb = (tid % TPR) * EPT;
    const bool lead = (tid % TPR) == 0;
    float sr[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) sr[i] = E.S[r * P + cb + i];
    __syncthreads();
    float* Hv = E.S;
    for (int k = 0; k < D - 2; ++k) {
      const int par = k & 1;
      if (r == k) {   // row k (= column k) as it stands
#pragma unroll
        for (int i = 0; i < EPT; i += 4) {
          floatx4_t v;
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = sr[i + u];
          *reinterpret_cast<floatx4_t*>(Hv + k * D + cb + i) = v;
        }
      }
      __syncthreads();
      if (w == 0) {   // the reflector of column k: v_k in place of row k
        float* hv = Hv + k * D;
        const float dk = hv[k], x0 = hv[k + 1];
        float xa[D / 64], sig = 0.0f;
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
          const int c = l + 64 * q;
          xa[q] = hv[c];
          sig = fmaf(c > k + 1 ? xa[q] : 0.0f, xa[q], sig);
        }
        sig = wave_sum_dpp(sig);
        float alpha = x0, bet = 0.0f;
        if (sig > 0.0f) {
          const float nrm = sqrtf(fmaf(x0, x0, sig));
          alpha = x0 >= 0.0f ? -nrm : nrm;
          bet = 1.0f / (nrm * (nrm + fabsf(x0)));
        }
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
          const int c = l + 64 * q;
          hv[c] = bet == 0.0f ? 0.0f : (c > k + 1 ? xa[q] : (c == k + 1 ? x0 - alpha : 0.0f));
        }
        if (l == 0) {
          E.d[k] = dk;
          E.e[k] = alpha;
          E.beta[k] = bet;
        }
      }
      __syncthreads();
      const float bet = E.beta[k];
      if (bet == 0.0f) continue;
      const float* hv = Hv + k * D;
      float pr = 0.0f;
#pragma unroll
      for (int i = 0; i < EPT; i += 4) {
        const floatx4_t v = *reinterpret_cast<const floatx4_t*>(hv + cb + i);
        pr = fmaf(sr[i], v[0], pr);
        pr = fmaf(sr[i + 1], v[1], pr);
        pr = fmaf(sr[i + 2], v[2], pr);
        pr = fmaf(sr[i + 3], v[3], pr);
      }
      pr = bet * group_sum<TPR>(pr);
      const float vr = hv[r];
      const float dv = wave_sum_dpp(lead ? vr * pr : 0.0f);
      if (l == 0) E.red[par * 4 + w] = dv;
      if (lead) E.pb[par * D + r] = pr;
      __syncthreads();
      const float K = 0.5f * bet * ((E.red[par * 4] + E.red[par * 4 + 1]) +
                                    (E.red[par * 4 + 2] + E.red[par * 4 + 3]));
      const float wr = fmaf(-K, vr, pr);
      const float* pp = E.pb + par * D + cb;
#pragma unroll
      for (int i = 0; i < EPT; i += 4) {
        const floatx4_t v = *reinterpret_cast<const floatx4_t*>(hv + cb + i);
        const floatx4_t pv = *reinterpret_cast<const floatx4_t*>(pp + i);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float wc = fmaf(-K, v[u], pv[u]);
          sr[i + u] -= fmaf(vr, wc, wr * v[u]);
        }
      }
    }
    if (r >= D - 2) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int c = cb + i;
        if (c == r) E.d[r] = sr[i];
        if (r == D - 1 && c == D - 2) E.e[D - 2] = sr[i];
      }
    }
    if (tid == 0) {
      E.e[D - 1] = 0.0f;
      E.beta[D - 2] = 0.0f;
      E.beta[D - 1] = 0.0f;
    }
    __syncthreads();
    if (tid < D) E.e2[tid] = E.e[tid] * E.e[tid];
    __syncthreads();
  }

  // --- Gershgorin interval and the scale of T --------------------------------
  float glo = INFINITY, ghi = -INFINITY, emax2 = 0.0f;
  for (int i = 0; i < D; ++i) {
    const float rad = (i > 0 ? fabsf(E.e[i - 1]) : 0.0f) + fabsf(E.e[i]);
    glo = fminf(glo, E.d[i] - rad);
    ghi = fmaxf(ghi, E.d[i] + rad);
    emax2 = fmaxf(emax2, E.e2[i]);
  }
  const float tnorm = fmaxf(fmaxf(fabsf(glo), fabsf(ghi)), 1e-30f);
  const float pivmin = 1.17549435e-38f * fmaxf(1.0f, emax2);

  // --- multisection: PPE lanes per eigenvalue -------------------------------
  {
    constexpr int PPE = 256 / D, LPE = 64 / PPE;
    const int j = w * LPE + l % LPE, m = l / LPE;
    float a = glo - 0x1p-20f * tnorm - pivmin, b = ghi + 0x1p-20f * tnorm + pivmin;
    const float tol = 0x1p-22f * tnorm;
    for (int it = 0; it < 48; ++it) {
      if (!(b - a > tol)) break;
      const float step = (b - a) * (1.0f / (float)(PPE + 1));
      const float x = fmaf((float)(m + 1), step, a);
      int cnt = 0;
      float q = E.d[0] - x;
      if (fabsf(q) < pivmin) q = -pivmin;
      cnt += q < 0.0f;
#pragma unroll 4
      for (int i = 1; i < D; ++i) {
        q = (E.d[i] - x) - E.e2[i - 1] * rcpf(q);
        if (fabsf(q) < pivmin) q = -pivmin;
        cnt += q < 0.0f;
      }
      float na = a, nb = b;
      int cms[PPE];
      if constexpr (PPE == 2) {   // the other half of the wave: v_permlane32_swap
        const auto sw = __builtin_amdgcn_permlane32_swap((uint32_t)cnt, (uint32_t)cnt, false, false);
        cms[0] = (int)sw[0];
        cms[1] = (int)sw[1];
      } else {
#pragma unroll
        for (int mm = 0; mm < PPE; ++mm) cms[mm] = __shfl(cnt, (l % LPE) + mm * LPE);
      }
#pragma unroll
      for (int mm = 0; mm < PPE; ++mm) {
        const int cm = cms[mm];
        const float xm = fmaf((float)(mm + 1), step, a);
        if (cm > j) nb = fminf(nb, xm); else na = fmaxf(na, xm);
      }
      if (na == a && nb == b) break;
      a = na;
      b = nb;
    }
    if (m == 0) lam[j] = 0.5f * (a + b);
  }
  __syncthreads();

  // --- inverse iteration: lane j < D, L in registers, x in LDS ---------------
  if (tid < D) {
    const int j = tid;
    const float mu = lam[j];
    const float piv = 0x1p-23f * tnorm;
    float* Zw = E.Zw;
    float Lr[D - 1];
    for (int i = 0; i < D; ++i) Zw[i * D + j] = ii_start(i, j);
#pragma unroll 1
    for (int it = 0; it < 3; ++it) {
      float dp = E.d[0] - mu;
      if (fabsf(dp) < piv) dp = piv;
      float rdp = rcpf(dp);
      float y = Zw[j];
      Zw[j] = y * rdp;
#pragma unroll
      for (int i = 0; i < D - 1; ++i) {
        const float li = E.e[i] * rdp;
        Lr[i] = li;
        dp = (E.d[i + 1] - mu) - li * E.e[i];
        if (fabsf(dp) < piv) dp = piv;
        rdp = rcpf(dp);
        const float bi = Zw[(i + 1) * D + j];
        y = fmaf(-li, y, bi);
        Zw[(i + 1) * D + j] = y * rdp;
      }
      float x = Zw[(D - 1) * D + j];
      float n2 = x * x;
#pragma unroll
      for (int i = D - 2; i >= 0; --i) {
        x = fmaf(-Lr[i], x, Zw[i * D + j]);
        Zw[i * D + j] = x;
        n2 = fmaf(x, x, n2);
      }
      const float inv = 1.0f / sqrtf(n2);
      for (int i = 0; i < D; ++i) Zw[i * D + j] *= inv;
    }
  }
  __syncthreads();

  // --- MGS and back-transform, one vector over PARTS lanes -------------------
  constexpr int PARTS = 256 / D, LPG = 64 / PARTS, CH = D / PARTS;
  const int j = w * LPG + (l % LPG), part = l / LPG, c0 = part * CH;
  auto reduce_parts = [&](float v) __attribute__((always_inline)) {
    if constexpr (LPG < 32) v += __shfl_xor(v, 16);
    return sum_halves(v);
  };
  float x[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) x[c] = E.Zw[(c0 + c) * D + j];
  for (int pass = 0; pass < 2; ++pass)   // twice: near-degenerate vectors leave the first
  for (int i = D - 1; i >= 0; --i) {     // pass only roughly orthogonal
    float* buf = E.xb + (i & 1) * D + c0;
    if (w == i / LPG) {
      float n2 = 0.0f;
#pragma unroll
      for (int c = 0; c < CH; ++c) n2 = fmaf(x[c], x[c], n2);
      const float inv = 1.0f / sqrtf(reduce_parts(n2));
      if (j == i) {
#pragma unroll
        for (int c = 0; c < CH; c += 4) {
          floatx4_t v;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            x[c + u] *= inv;
            v[u] = x[c + u];
          }
          *reinterpret_cast<floatx4_t*>(buf + c) = v;
        }
      }
    }
    __syncthreads();
    if (j < i) {
      floatx4_t bv[CH / 4];
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < CH; c += 4) {
        bv[c / 4] = *reinterpret_cast<const floatx4_t*>(buf + c);
#pragma unroll
        for (int u = 0; u < 4; ++u) dot = fmaf(x[c + u], bv[c / 4][u], dot);
      }
      dot = reduce_parts(dot);
#pragma unroll
      for (int c = 0; c < CH; c += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) x[c + u] = fmaf(-dot, bv[c / 4][u], x[c + u]);
    }
  }
  for (int k = D - 3; k >= 0; --k) {
    const float bet = E.beta[k];
    if (bet == 0.0f) continue;
    const float* v = E.S + k * D + c0;
    floatx4_t vv[CH / 4];
    float dot = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; c += 4) {
      vv[c / 4] = *reinterpret_cast<const floatx4_t*>(v + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) dot = fmaf(vv[c / 4][u], x[c + u], dot);
    }
    dot = bet * reduce_parts(dot);
#pragma unroll
    for (int c = 0; c < CH; c += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u) x[c + u] = fmaf(-dot, vv[c / 4][u], x[c + u]);
  }
#pragma unroll
  for (int c = 0; c < CH; c += 4) {
    floatx4_t v;
    v[0] = x[c]; v[1] = x[c + 1]; v[2] = x[c + 2]; v[3] = x[c + 3];
    *reinterpret_cast<floatx4_t*>(Xv + (int64_t)j * D + c0 + c) = v;
  }
  __threadfence_block();
  __syncthreads();
}

// C = A Bt^T on 256 threads: C[i][n] = sum_k A[i][k] Bt[n][k], both operands
// in LDS with pitch D + 4 (16-byte rows, read four k at a time; the 16 Bt rows
// a wave reads fall on disjoint banks). Each thread owns a (D/16) x (D/16)
// block: rows ty + 16 m, columns tx + 16 n.
template <int D>
CA_DEV void matmul_nt(const float* A, const float* Bt, float* C, int ldc) {
  constexpr int TM = D / 16, PM = D + 4;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[TM][TM];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TM; ++n) acc[m][n] = 0.0f;
  for (int k = 0; k < D; k += 4) {
    floatx4_t a[TM], b[TM];
#pragma unroll
    for (int m = 0; m < TM; ++m) a[m] = *reinterpret_cast<const floatx4_t*>(A + (ty + 16 * m) * PM + k);
#pragma unroll
    for (int n = 0; n < TM; ++n) b[n] = *reinterpret_cast<const floatx4_t*>(Bt + (tx + 16 * n) * PM + k);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TM; ++n) acc[m][n] = fmaf(a[m][u], b[n][u], acc[m][n]);
  }
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TM; ++n) C[(int64_t)(ty + 16 * m) * ldc + tx + 16 * n] = acc[m][n];
}

// dst (pitch D + 4) = src (pitch D), or its transpose
template <int D, bool TRANS>
CA_DEV void load_nt(float* dst, const float* src) {
  constexpr int PM = D + 4;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int i = e / D, k = e % D;
    if (TRANS) dst[k * PM + i] = src[e];
    else dst[i * PM + k] = src[e];
  }
}

// dst[i][k] (pitch D + 1, LDS) = scale_i src[i][k] (pitch D)
template <int D>
CA_DEV void load_mat(float* dst, const float* src, const float* scale) {
  constexpr int P = D + 1;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int i = e / D, k = e % D;
    dst[i * P + k] = scale ? scale[i] * src[e] : src[e];
  }
}

CA_DEV void block_sync_global() {
  __threadfence_block();
  __syncthreads();
}

template <int D>
struct BasisLds {
  static constexpr int P = D + 1;
  static constexpr int R1 = D * (D + 4);   // also holds a pitch-(D + 4) matmul operand
  static constexpr int R2 = D * (D + 4);
  static constexpr int SMALL = 12 * D + 16;
  static constexpr size_t bytes = (size_t)(R1 + R2 + SMALL) * 4;
};

// Pivoted Cholesky factor M = F F^T of a symmetric PSD D x D matrix (in LDS,
// pitch D + 1), right-looking with the rows in registers (TPR threads per
// row). Step k pivots on the largest remaining diagonal entry p_k, so a
// singular metric's range is taken first with large
// pivots; the factor stops at the first pivot at or below 2^-20 of the
// largest diagonal entry (what remains is rounding noise of the null space).
// (Among equal largest entries the one held by the lowest lane is taken.)
// Column k of F (row k of F^T) is lsc[k] Lraw[k][c] for every c not pivoted
// before step k (step_of[c] >= k), zero elsewhere; lsc[k] = 0 past the stop.
template <int D>
CA_DEV void cholesky_rows(const float* S, float* rb, float* diag, int* step_of, int* sel,
                          float* lsc, float* __restrict__ Lraw) {
  constexpr int P = D + 1, TPR = 256 / D, EPT = D / TPR, DL = D / 64;
  const int tid = threadIdx.x, r = tid / TPR, cb = (tid % TPR) * EPT;
  const int w = tid >> 6, l = tid & 63;
  float sr[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) sr[i] = S[r * P + cb + i];
  float dmax = 0.0f;
  for (int i = 0; i < D; ++i) dmax = fmaxf(dmax, S[i * P + i]);
  const float tolp = 0x1p-20f * dmax;
  // wave 0: argmax of the remaining diagonal (the lowest index on ties)
  auto pick = [&](int slot) __attribute__((always_inline)) {
    float best = -INFINITY;
    int bi = D;
#pragma unroll
    for (int q = 0; q < DL; ++q) {
      const int c = l + 64 * q;
      if (step_of[c] == D && diag[c] > best) { best = diag[c]; bi = c; }
    }
    const float m = wave_max_dpp(best);
    const uint64_t hit = __ballot(bi < D && best == m);
    const int src = hit ? (int)__builtin_ctzll(hit) : 0;
    const int pb = hit ? __builtin_amdgcn_readlane(bi, src) : D;
    if (l == 0) sel[slot] = pb;
  };
  if (w == 0) {
#pragma unroll
    for (int q = 0; q < DL; ++q) {
      const int c = l + 64 * q;
      diag[c] = S[c * P + c];
      step_of[c] = D;
    }
    __builtin_amdgcn_wave_barrier();
    pick(0);
  }
  if (tid < D) lsc[tid] = 0.0f;
  __syncthreads();
  for (int k = 0; k < D; ++k) {
    const int p = sel[k & 1];
    if (p >= D) break;
    if (r == p) {
#pragma unroll
      for (int i = 0; i < EPT; i += 4) {
        floatx4_t v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = sr[i + u];
        *reinterpret_cast<floatx4_t*>(rb + cb + i) = v;
        *reinterpret_cast<floatx4_t*>(Lraw + (int64_t)k * D + cb + i) = v;
      }
    }
    __syncthreads();
    const float piv = rb[p];
    if (!(piv > tolp)) break;
    const float rr = rb[r] / piv;
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(rb + cb + i);
#pragma unroll
      for (int u = 0; u < 4; ++u) sr[i + u] = fmaf(-rr, v[u], sr[i + u]);
    }
    if (w == 0) {
      if (l == 0) {
        lsc[k] = 1.0f / sqrtf(piv);
        step_of[p] = k;
      }
      const float ip = 1.0f / piv;
#pragma unroll
      for (int q = 0; q < DL; ++q) {
        const int c = l + 64 * q;
        const float v = rb[c];
        diag[c] = fmaf(-v * ip, v, diag[c]);
      }
      __builtin_amdgcn_wave_barrier();
      pick((k + 1) & 1);
    }
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
}

// dst (pitch D + 4) = F^T (row k = column k of F), or F itself when TRANS
template <int D, bool TRANS>
CA_DEV void load_lt(float* dst, const float* Lraw, const float* lsc, const int* step_of) {
  constexpr int PM = D + 4;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int k = e / D, c = e % D;
    const float v = (lsc[k] != 0.0f && step_of[c] >= k) ? lsc[k] * Lraw[e] : 0.0f;
    if (TRANS) dst[c * PM + k] = v;
    else dst[k * PM + c] = v;
  }
}

// One workgroup per tree (2 bh + tensor; tensor 0 = queries, 1 = keys).
// Geometry M: M_k for queries, M_q for keys (identity without the transform);
// covariance C_x of the representation: C_q (queries), M_k (keys).
//   M = F F^T (pivoted Cholesky);  Z = F^T C_x F;  eig(Z) -> W;  a_j = F w_j.
// Any factor F F^T = M gives the same a_j up to sign (for invertible M the
// eigenvectors of F^T C_x F are those of R C_x R, R the symmetric root,
// rotated by the orthogonal F^T R^-1), so the root is not formed. Each a_j is signed so that its
// largest-magnitude entry (the first on ties) is positive; output row D-1-j is
// a_j for the (j+1)-th smallest eigenvalue, so the rows descend.
template <int D>
__global__ __launch_bounds__(256) void basis_kernel(const float* __restrict__ Mq,
                                                    const float* __restrict__ Mk,
                                                    const float* __restrict__ Cq, int transform,
                                                    float* __restrict__ Rbuf,
                                                    float* __restrict__ Zbuf,
                                                    float* __restrict__ At) {
  using L = BasisLds<D>;
  constexpr int P = L::P;
  extern __shared__ __attribute__((aligned(16))) float bsm[];
  float* r1 = bsm;
  float* r2 = bsm + L::R1;
  float* sm = r2 + L::R2;
  EigLds<D> E;
  E.S = r1;
  E.Zw = r2;
  E.d = sm;
  E.e = sm + D;
  E.e2 = sm + 2 * D;
  E.beta = sm + 3 * D;
  E.pb = sm + 4 * D;            // [2 D]
  E.xb = sm + 6 * D;            // [2 D]
  float* lam = sm + 8 * D;
  float* lsc = sm + 9 * D;
  E.red = sm + 10 * D;          // [8]
  int* step_of = reinterpret_cast<int*>(sm + 11 * D);   // [D]
  int* sel = reinterpret_cast<int*>(sm + 12 * D);       // [2]
  const int tree = blockIdx.x, bh = tree >> 1, tensor = tree & 1;
  const int tid = threadIdx.x;
  const float* Cx = (tensor == 0 ? Cq : Mk) + (int64_t)bh * D * D;
  float* Lraw = Rbuf + (int64_t)tree * D * D;
  float* Z = Zbuf + (int64_t)tree * D * D;   // scratch: F^T C_x, Z, then W, then the a_j
  float* out = At + (int64_t)tree * D * D;

  if (transform) {
    const float* M = (tensor == 0 ? Mk : Mq) + (int64_t)bh * D * D;
    load_mat<D>(r1, M, nullptr);
    __syncthreads();
    cholesky_rows<D>(r1, E.pb, E.d, step_of, sel, lsc, Lraw);
    load_lt<D, false>(r1, Lraw, lsc, step_of);
    load_nt<D, false>(r2, Cx);
    __syncthreads();
    matmul_nt<D>(r1, r2, Z, D);   // T = F^T C_x (C_x symmetric)
    block_sync_global();
    load_nt<D, false>(r2, Z);
    __syncthreads();
    matmul_nt<D>(r2, r1, Z, D);   // Z = T F
    block_sync_global();
    load_mat<D>(r1, Z, nullptr);
  } else {
    load_mat<D>(r1, Cx, nullptr);
  }
  __syncthreads();
  eig_sym<D>(E, lam, Z);   // row j of Z: w_j
  if (transform) {
    load_nt<D, false>(r1, Z);
    load_lt<D, true>(r2, Lraw, lsc, step_of);
    __syncthreads();
    matmul_nt<D>(r1, r2, Z, D);   // row j: w_j^T F^T = (F w_j)^T
    block_sync_global();
  }
  // sign and order: TPR threads per row
  {
    constexpr int TPR = 256 / D, EPT = D / TPR;
    const int j = tid / TPR, cb = (tid % TPR) * EPT;
    const float* zr = Z + (int64_t)j * D + cb;
    float best = -1.0f, sv = 1.0f;
    int bi = 0;
    for (int i = 0; i < EPT; ++i) {
      const float v = zr[i];
      if (fabsf(v) > best) { best = fabsf(v); bi = cb + i; sv = v; }
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      const float ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      const float os = __shfl_xor(sv, o);
      if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; sv = os; }
    }
    const float sg = sv < 0.0f ? -1.0f : 1.0f;
    float* orow = out + (int64_t)(D - 1 - j) * D + cb;
    for (int i = 0; i < EPT; ++i) orow[i] = sg * zr[i];
  }
}

template <int D>
void launch_basis_d(const void* Q, int dtype, int BH, int N, int transform, const float* s,
                    const float* Mq, const float* Mk, float* partial, float* Cq, float* Rbuf,
                    float* Zbuf, float* At, hipStream_t st) {
  const int rows = metric_rows_per_chunk(N, BH);
  const int nchunks = (N + rows - 1) / rows;
  dim3 gp(nchunks, BH);
  if (dtype == 0)
    qmoment_partial_bf16<D><<<gp, 256, 0, st>>>((const uint16_t*)Q, s, N, rows, nchunks, partial);
  else
    qmoment_partial_f32<D><<<gp, 256, 0, st>>>((const float*)Q, s, N, rows, nchunks, partial);
  dim3 gr((D * D + 255) / 256, BH);
  qmoment_reduce<D><<<gr, 256, 0, st>>>(partial, nchunks, N, Cq);
  constexpr size_t sm = BasisLds<D>::bytes;
  CA_MAX_LDS_ONCE(&basis_kernel<D>, sm);
  basis_kernel<D><<<2 * BH, 256, sm, st>>>(Mq, Mk, Cq, transform, Rbuf, Zbuf, At);
}

// ----------------------------------------------------------------------------
// Rotation of every vector into its tree's basis once (the diagonalized
// splitting then only reads coordinates): Y[tree][t][j] = x_t . a_j, with
// x = s q for queries and x = k for keys, fp32 [2 BH][N][D].
// ----------------------------------------------------------------------------

// Three-term bf16 split of At (hi + mid + lo carries 24 significant bits):
// At3 [2 BH][3][D][D].
template <int D>
__global__ __launch_bounds__(256) void basis_split(const float* __restrict__ At, int trees,
                                                   uint16_t* __restrict__ At3) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)trees * D * D) return;
  const int64_t tree = e / (D * D), r = e % (D * D);
  const float g = At[e];
  const uint16_t hi = f32_to_bf16(g);
  const float r1 = g - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r1);
  const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
  uint16_t* o = At3 + tree * 3 * D * D + r;
  o[0] = hi;
  o[D * D] = mid;
  o[2 * D * D] = lo;
}

constexpr int kRotThreads = 1024;   // 16 waves, one 32-token block each
constexpr int kRotTokens = 2048;    // tokens per workgroup

// bf16 rows on MFMA: the three bf16 terms of the tree's basis sit in LDS;
// each wave takes 32-token blocks in turn (the B operand, the bf16 rows,
// exact, read from global memory two blocks ahead) and forms every
// coordinate block from them. Lane (r, h) ends with coordinates
// 32 bn + 8 g + 4 h + (0..3) of token t0 + r and stores them as 16-byte
// vectors.
template <int D>
__global__ __launch_bounds__(kRotThreads) void rotate_bf16(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const float* __restrict__ s,
                                                           const uint16_t* __restrict__ At3, int N,
                                                           float* __restrict__ Y, int kvg) {
  constexpr int NB = D / 32, KS = D / 16, PB = D + 8, NW = kRotThreads / 64;
  extern __shared__ __attribute__((aligned(16))) uint16_t sb[];   // [3 D][PB]
  const int tree = blockIdx.y, bh = tree >> 1, tensor = tree & 1;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 31, h = l >> 5;
  {
    const uint16_t* src = At3 + (int64_t)tree * 3 * D * D;
    for (int e = tid; e < 3 * D * D / 8; e += kRotThreads) {
      const int row = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<u32x4_t*>(&sb[row * PB + 8 * c8]) =
          *reinterpret_cast<const u32x4_t*>(src + (int64_t)row * D + 8 * c8);
    }
  }
  __syncthreads();
  const uint16_t* X = tensor == 0 ? Q + (int64_t)bh * N * D : K + (int64_t)(bh / kvg) * N * D;
  const float* sv = tensor == 0 ? s + (int64_t)bh * N : nullptr;
  float* Yt = Y + (int64_t)tree * N * D;
  const int tend = min(N, (blockIdx.x + 1) * kRotTokens);
  auto load = [&](int t0, u32x4_t* av, float* sc) __attribute__((always_inline)) {
    const int tok = t0 + r;
    const bool ok = tok < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      av[ks] = ok ? *reinterpret_cast<const u32x4_t*>(X + (int64_t)tok * D + 16 * ks + 8 * h)
                  : u32x4_t{0u, 0u, 0u, 0u};
    *sc = ok && sv ? sv[tok] : 1.0f;
  };
  constexpr int STR = 32 * NW;
  int t0 = blockIdx.x * kRotTokens + 32 * w;
  if (t0 >= tend) return;
  u32x4_t a0[KS], a1[KS];   // blocks t0 and t0 + STR in flight
  float s0, s1;
  load(t0, a0, &s0);
  load(t0 + STR, a1, &s1);
  for (; t0 < tend; t0 += STR) {
    const int tok = t0 + r;
#pragma unroll 1
    for (int bn = 0; bn < NB; ++bn) {   // not unrolled: the basis operands stay in LDS
      floatx16_t acc0 = zero16(), acc1 = zero16();   // two chains: even and odd k-steps
      const uint16_t* bb = sb + (32 * bn + r) * PB + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KS; ks += 2)
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(bb + t * D * PB + 16 * ks);
          const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(bb + t * D * PB + 16 * ks + 16);
          acc0 = mfma32(b0, as_bf16x8(a0[ks]), acc0);
          acc1 = mfma32(b1, as_bf16x8(a0[ks + 1]), acc1);
        }
      if (tok < N) {
        float* yr = Yt + (int64_t)tok * D + 32 * bn + 4 * h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          floatx4_t v;
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = s0 * (acc0[4 * g + u] + acc1[4 * g + u]);
          *reinterpret_cast<floatx4_t*>(yr + 8 * g) = v;
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a0[ks] = a1[ks];
    s0 = s1;
    if (t0 + 2 * STR < tend) load(t0 + 2 * STR, a1, &s1);
  }
}

// fp32 rows on the VALU: thread (j, g) holds a_j and sums rows g, g + G, ...
// of a 32-token tile staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void rotate_f32(const float* __restrict__ Q,
                                                  const float* __restrict__ K,
                                                  const float* __restrict__ s,
                                                  const float* __restrict__ At, int N,
                                                  float* __restrict__ Y, int kvg) {
  constexpr int G = 256 / D, TT = 32;
  __shared__ float sx[TT][D + 1];
  const int tree = blockIdx.y, bh = tree >> 1, tensor = tree & 1;
  const int tid = threadIdx.x, j = tid % D, g = tid / D;
  const float* X = tensor == 0 ? Q + (int64_t)bh * N * D : K + (int64_t)(bh / kvg) * N * D;
  const float* sv = tensor == 0 ? s + (int64_t)bh * N : nullptr;
  float aj[D];
#pragma unroll
  for (int k = 0; k < D; ++k) aj[k] = At[((int64_t)tree * D + j) * D + k];
  const int t0 = blockIdx.x * TT;
  for (int e = tid; e < TT * D; e += 256) {
    const int t = e / D, k = e % D;
    sx[t][k] = t0 + t < N ? X[(int64_t)(t0 + t) * D + k] : 0.0f;
  }
  __syncthreads();
  for (int t = g; t < TT; t += G) {
    if (t0 + t >= N) break;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) acc = fmaf(sx[t][k], aj[k], acc);
    Y[((int64_t)tree * N + t0 + t) * D + j] = (sv ? sv[t0 + t] : 1.0f) * acc;
  }
}

template <int D>
void launch_rotate_d(const void* Q, const void* K, int dtype, int BH, int N, const float* s,
                     const float* At, uint16_t* At3, float* Y, int kvg, hipStream_t st) {
  const int trees = 2 * BH;
  if (dtype == 0) {
    basis_split<D><<<(unsigned)(((int64_t)trees * D * D + 255) / 256), 256, 0, st>>>(At, trees, At3);
    dim3 g((N + kRotTokens - 1) / kRotTokens, trees);
    constexpr size_t sm = (size_t)3 * D * (D + 8) * 2;
    CA_MAX_LDS_ONCE(&rotate_bf16<D>, sm);
    rotate_bf16<D><<<g, kRotThreads, sm, st>>>((const uint16_t*)Q, (const uint16_t*)K, s, At3, N, Y, kvg);
  } else {
    dim3 g((N + 31) / 32, trees);
    rotate_f32<D><<<g, 256, 0, st>>>((const float*)Q, (const float*)K, s, At, N, Y, kvg);
  }
}

}  // namespace

void launch_basis(const void* Q, int dtype, int BH, int N, int D, int transform, const float* s,
                  const float* Mq, const float* Mk, float* partial, float* Cq, float* Rbuf,
                  float* Zbuf, float* At, hipStream_t st) {
  if (D == 64) launch_basis_d<64>(Q, dtype, BH, N, transform, s, Mq, Mk, partial, Cq, Rbuf, Zbuf, At, st);
  else launch_basis_d<128>(Q, dtype, BH, N, transform, s, Mq, Mk, partial, Cq, Rbuf, Zbuf, At, st);
}

void launch_rotate(const void* Q, const void* K, int dtype, int BH, int N, int D, const float* s,
                   const float* At, uint16_t* At3, float* Y, int kvg, hipStream_t st) {
  if (D == 64) launch_rotate_d<64>(Q, K, dtype, BH, N, s, At, At3, Y, kvg, st);
  else launch_rotate_d<128>(Q, K, dtype, BH, N, s, At, At3, Y, kvg, st);
}

}  // namespace ca
