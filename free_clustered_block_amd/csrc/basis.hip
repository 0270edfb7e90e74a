// Principal-component basis for diagonalized recursive splitting (paper v1
// §3.2.1 "Diagonalized recursive splitting"; later revision §4.1.1): the
// vectors of each tree are rotated once into the principal-component basis of
// the whole set, taken in the transform's geometry (z = R x, R the root matrix
// of the metric, v1 §3.2.2), and every node then splits along the coordinate
// of highest sample variance.
//
//   qmoment_partial / qmoment_reduce   C_q = Cov(s q) over all queries (the
//       query representation x = s q of Eq. 16); the key covariance is M_k of
//       the metric pass.
//   basis_kernel   one workgroup per tree: cyclic Jacobi eigendecomposition of
//       the geometry M (-> symmetric root R, negative eigenvalues clamped),
//       Z = R C_x R, Jacobi of Z (-> W, lam), columns ordered by descending
//       eigenvalue and signed so that each column's largest-magnitude entry is
//       positive; writes A^T with A = R W, so row j of the output is the
//       direction whose projection x . a_j is coordinate j.
#include "kernels.h"
#include "mfma.h"

namespace ca {

namespace {

constexpr int kMomTile = 128;   // tokens per LDS tile of the bf16 moment pass

// Weighted second moment sum_t w_t q_t q_t^T (w = s^2) and sum_t s_t q_t over
// a chunk of query rows, on bf16 MFMA: the A operand is q (exact in bf16), the
// B operand w q split into three bf16 terms (fp32 accuracy).
template <int D>
__global__ __launch_bounds__(256) void qmoment_partial_bf16(const uint16_t* __restrict__ Q,
                                                            const float* __restrict__ s, int N,
                                                            int rows_per_chunk, int nchunks,
                                                            float* __restrict__ partial) {
  constexpr int TT = kMomTile;
  constexpr int NB = D / 32;
  constexpr int BPW = NB * NB / 4;          // 32x32 blocks per wave
  constexpr int LDT = TT + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sx[D][LDT];
  __shared__ float sw[TT], sv[TT];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int r0 = chunk * rows_per_chunk, r1 = min(N, r0 + rows_per_chunk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, r = l & 31;
  const uint16_t* X = Q + (int64_t)bh * N * D;
  const float* sq = s + (int64_t)bh * N;
  floatx16_t acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) acc[i] = zero16();
  float s1 = 0.0f;   // sum of s q over dim tid (tid < D), in token order
  for (int base = r0; base < r1; base += TT) {
    // tile into LDS transposed: element (token t, dim d) -> sx[d][t]
    for (int e = tid; e < TT * D / 2; e += 256) {
      const int t = e / (D / 2), d2 = e % (D / 2);
      uint32_t v = 0u;
      if (base + t < r1) v = *reinterpret_cast<const uint32_t*>(X + (int64_t)(base + t) * D + 2 * d2);
      sx[2 * d2][t] = (uint16_t)(v & 0xFFFFu);
      sx[2 * d2 + 1][t] = (uint16_t)(v >> 16);
    }
    if (tid < TT) {
      const float st = base + tid < r1 ? sq[base + tid] : 0.0f;
      sw[tid] = st * st;
      sv[tid] = st;
    }
    __syncthreads();
    if (tid < D) {
      const int nt = min(TT, r1 - base);
      for (int t = 0; t < nt; ++t) s1 = fmaf(sv[t], bf16_to_f32(sx[tid][t]), s1);
    }
#pragma unroll 1
    for (int ks = 0; ks < TT / 16; ++ks) {
      const int k0 = 16 * ks + 8 * h;
      float wk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wk[e] = sw[k0 + e];
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int b = w * BPW + i, bm = b / NB, bn = b % NB;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sx[bm * 32 + r][k0]);
        const u32x4_t bw = *reinterpret_cast<const u32x4_t*>(&sx[bn * 32 + r][k0]);
        const uint32_t bb[4] = {bw.x, bw.y, bw.z, bw.w};
        float hi[8], mid[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = bf16_to_f32((uint16_t)((bb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu)) * wk[e];
          hi[e] = (float)(__bf16)v;
          const float rem = v - hi[e];
          mid[e] = (float)(__bf16)rem;
          lo[e] = rem - mid[e];
        }
        acc[i] = mfma32(a, as_bf16x8(pack8(hi)), acc[i]);
        acc[i] = mfma32(a, as_bf16x8(pack8(mid)), acc[i]);
        acc[i] = mfma32(a, as_bf16x8(pack8(lo)), acc[i]);
      }
    }
    __syncthreads();
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
// Cyclic Jacobi on a symmetric D x D matrix in LDS (row pitch D + 1), all 256
// threads: each round applies D/2 disjoint rotations of the round-robin
// (circle-method) pairing, rows first then columns; a rotation is skipped when
// |a_pq| <= max(1e-7 sqrt(|a_pp a_qq|), 2^-26 tr|S|) with tr|S| the sum of the
// diagonal magnitudes on entry (below the rounding of fp32 entries, so sweeps
// end even where small eigenvalues sit next to large ones); sweeps stop when a
// whole sweep skipped every rotation, after at most kMaxSweeps. V accumulates the
// rotations (V <- V J): its columns are the eigenvectors, S's diagonal the
// eigenvalues.
// ----------------------------------------------------------------------------

constexpr int kMaxSweeps = 30;

template <int D>
struct JacobiLds {
  static constexpr int P = D + 1;
  float* S;      // [D][P]
  float* V;      // [D][P]
  float* cs;     // [D/2][2]
  int* pq;       // [D/2][2]
  int* flag;     // [0]: rotations done in the sweep; [1]: absolute threshold (float bits)
};

// pair i of round r (0 <= r < D - 1) of the circle method on D players
CA_DEV void jacobi_pair(int D, int r, int i, int* p, int* q) {
  int a, b;
  if (i == 0) {
    a = D - 1;
    b = r;
  } else {
    a = (r + i) % (D - 1);
    b = (r - i + D - 1) % (D - 1);
  }
  *p = min(a, b);
  *q = max(a, b);
}

template <int D>
CA_DEV void jacobi(const JacobiLds<D>& J) {
  constexpr int P = JacobiLds<D>::P, H = D / 2;
  const int tid = threadIdx.x;
  for (int e = tid; e < D * D; e += 256) J.V[(e / D) * P + e % D] = (e / D == e % D) ? 1.0f : 0.0f;
  if (tid == 0) {
    float tr = 0.0f;
    for (int i = 0; i < D; ++i) tr += fabsf(J.S[i * P + i]);
    J.flag[1] = __float_as_int(tr * 0x1p-26f);
  }
  __syncthreads();
  const float tol_abs = __int_as_float(J.flag[1]);
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    if (tid == 0) *J.flag = 0;
    __syncthreads();
    for (int rd = 0; rd < D - 1; ++rd) {
      if (tid < H) {
        int p, q;
        jacobi_pair(D, rd, tid, &p, &q);
        const float app = J.S[p * P + p], aqq = J.S[q * P + q], apq = J.S[p * P + q];
        float c = 1.0f, sn = 0.0f;
        if (fabsf(apq) > fmaxf(1e-7f * sqrtf(fabsf(app) * fabsf(aqq)), tol_abs) && apq != 0.0f) {
          const float th = (aqq - app) / (2.0f * apq);
          const float t = (th >= 0.0f ? 1.0f : -1.0f) / (fabsf(th) + sqrtf(th * th + 1.0f));
          c = 1.0f / sqrtf(t * t + 1.0f);
          sn = t * c;
          *J.flag = 1;
        }
        J.cs[2 * tid] = c;
        J.cs[2 * tid + 1] = sn;
        J.pq[2 * tid] = p;
        J.pq[2 * tid + 1] = q;
      }
      __syncthreads();
      // rows: S <- J^T S
      for (int e = tid; e < H * D; e += 256) {
        const int i = e / D, k = e % D;
        const float c = J.cs[2 * i], sn = J.cs[2 * i + 1];
        if (sn == 0.0f) continue;
        const int p = J.pq[2 * i], q = J.pq[2 * i + 1];
        const float sp = J.S[p * P + k], sq = J.S[q * P + k];
        J.S[p * P + k] = c * sp - sn * sq;
        J.S[q * P + k] = sn * sp + c * sq;
      }
      __syncthreads();
      // columns: S <- S J, V <- V J; the rotated pair's off-diagonal is zero
      for (int e = tid; e < H * D; e += 256) {
        const int i = e / D, k = e % D;
        const float c = J.cs[2 * i], sn = J.cs[2 * i + 1];
        if (sn == 0.0f) continue;
        const int p = J.pq[2 * i], q = J.pq[2 * i + 1];
        const float sp = J.S[k * P + p], sq = J.S[k * P + q];
        float np = c * sp - sn * sq, nq = sn * sp + c * sq;
        if (k == q) np = 0.0f;
        if (k == p) nq = 0.0f;
        J.S[k * P + p] = np;
        J.S[k * P + q] = nq;
        const float vp = J.V[k * P + p], vq = J.V[k * P + q];
        J.V[k * P + p] = c * vp - sn * vq;
        J.V[k * P + q] = sn * vp + c * vq;
      }
      __syncthreads();
    }
    const int done = *J.flag == 0;
    __syncthreads();
    if (done) break;
  }
}

// One workgroup per tree (2 bh + tensor; tensor 0 = queries, 1 = keys).
// Geometry M: M_k for queries, M_q for keys (identity without the transform);
// covariance C_x of the representation: C_q (queries), M_k (keys).
template <int D>
__global__ __launch_bounds__(256) void basis_kernel(const float* __restrict__ Mq,
                                                    const float* __restrict__ Mk,
                                                    const float* __restrict__ Cq, int transform,
                                                    float* __restrict__ Rbuf,
                                                    float* __restrict__ Zbuf,
                                                    float* __restrict__ At) {
  constexpr int P = D + 1;
  extern __shared__ __attribute__((aligned(16))) float bsm[];
  JacobiLds<D> J;
  J.S = bsm;
  J.V = bsm + D * P;
  J.cs = bsm + 2 * D * P;
  float* lam = J.cs + D;                     // [D]
  float* sgn = lam + D;                      // [D]
  int* rank = reinterpret_cast<int*>(sgn + D);
  J.pq = rank + D;
  J.flag = J.pq + D;
  const int tree = blockIdx.x, bh = tree >> 1, tensor = tree & 1;
  const int tid = threadIdx.x;
  const float* Cx = (tensor == 0 ? Cq : Mk) + (int64_t)bh * D * D;
  float* R = Rbuf + (int64_t)tree * D * D;
  float* Z = Zbuf + (int64_t)tree * D * D;

  // R: symmetric root of the geometry
  if (transform) {
    const float* M = (tensor == 0 ? Mk : Mq) + (int64_t)bh * D * D;
    for (int e = tid; e < D * D; e += 256) J.S[(e / D) * P + e % D] = M[e];
    __syncthreads();
    jacobi<D>(J);
    if (tid < D) lam[tid] = sqrtf(fmaxf(J.S[tid * P + tid], 0.0f));
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) {
      const int k = e / D, l = e % D;
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) acc = fmaf(J.V[k * P + i] * lam[i], J.V[l * P + i], acc);
      J.S[k * P + l] = acc;   // S is free after the eigenvalues were read
    }
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) R[e] = J.S[(e / D) * P + e % D];
    // T = C_x R into V, then Z = R T to global memory
    for (int e = tid; e < D * D; e += 256) {
      const int k = e / D, l = e % D;
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) acc = fmaf(Cx[(int64_t)k * D + i], J.S[i * P + l], acc);
      J.V[k * P + l] = acc;
    }
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) {
      const int k = e / D, l = e % D;
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) acc = fmaf(J.S[k * P + i], J.V[i * P + l], acc);
      Z[e] = acc;
    }
    __threadfence_block();
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) J.S[(e / D) * P + e % D] = Z[e];
  } else {
    for (int e = tid; e < D * D; e += 256) {
      R[e] = (e / D == e % D) ? 1.0f : 0.0f;
      J.S[(e / D) * P + e % D] = Cx[e];
    }
  }
  __threadfence_block();
  __syncthreads();
  // W, lam of Z = R C_x R
  jacobi<D>(J);
  if (tid < D) lam[tid] = J.S[tid * P + tid];
  __syncthreads();
  if (tid < D) {
    // descending eigenvalue order (ties to the lower index) and the sign that
    // makes the column's largest-magnitude entry (the first on ties) positive
    const float li = lam[tid];
    int rk = 0;
    for (int j = 0; j < D; ++j) rk += (lam[j] > li) || (lam[j] == li && j < tid);
    rank[tid] = rk;
    int kb = 0;
    float best = -1.0f;
    for (int k = 0; k < D; ++k) {
      const float v = fabsf(J.V[k * P + tid]);
      if (v > best) { best = v; kb = k; }
    }
    sgn[tid] = J.V[kb * P + tid] < 0.0f ? -1.0f : 1.0f;
  }
  __syncthreads();
  // A = R W: row rank[i] of A^T is sign_i (R w_i)
  float* out = At + (int64_t)tree * D * D;
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, k = e % D;   // eigenvector i, component k
    float acc = 0.0f;
    for (int l = 0; l < D; ++l) acc = fmaf(R[(int64_t)k * D + l], J.V[l * P + i], acc);
    out[(int64_t)rank[i] * D + k] = sgn[i] * acc;
  }
}

template <int D>
constexpr size_t basis_smem() {
  return (size_t)(2 * D * (D + 1) + 3 * D + D) * 4 + (size_t)(D + D + 4) * 4;
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
  constexpr size_t sm = basis_smem<D>();
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&basis_kernel<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    attr_set = true;
  }
  basis_kernel<D><<<2 * BH, 256, sm, st>>>(Mq, Mk, Cq, transform, Rbuf, Zbuf, At);
}

}  // namespace

void launch_basis(const void* Q, int dtype, int BH, int N, int D, int transform, const float* s,
                  const float* Mq, const float* Mk, float* partial, float* Cq, float* Rbuf,
                  float* Zbuf, float* At, hipStream_t st) {
  if (D == 64) launch_basis_d<64>(Q, dtype, BH, N, transform, s, Mq, Mk, partial, Cq, Rbuf, Zbuf, At, st);
  else launch_basis_d<128>(Q, dtype, BH, N, transform, s, Mq, Mk, partial, Cq, Rbuf, Zbuf, At, st);
}

}  // namespace ca
