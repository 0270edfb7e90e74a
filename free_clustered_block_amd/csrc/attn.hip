// Block-sparse attention with striped mean-compensation (paper v1 §1.2
// Eq. 2 and 5-6, App. A Eq. 21-22; the kernel returns the softmax denominator
// as in §3.1) and the dense baseline (Eq. 1), on gfx950 bf16 MFMA.
//
// bf16 path:
//   permute_kv   one workgroup per key cluster: gathers the cluster's K rows
//                into a contiguous zero-padded tile [c][D], its V rows into
//                transposed sub-tiles [c/64][D][64] (key order swizzled to the
//                MFMA operand order), and forms the key/value centroids and
//                ln n_c.
//   attn_fwd     one workgroup per query cluster (c/32 waves, 32 queries per
//                wave): the selected key clusters stream through LDS in
//                double-buffered sub-tiles of 64 keys, S^T = K Q^T and
//                O^T += V^T P^T run on
//                v_mfma_f32_32x32x16_bf16 with an fp32 online softmax (exp2);
//                the excluded clusters then enter through their centroids,
//                streamed the same way as sub-tiles of 64 centroids (bf16
//                kbar rows as keys, vbar as values, logit scale q.kbar +
//                ln n_c, -inf for selected or padding clusters) in the same
//                running maximum and sum. O is scattered back to token order.
// FP8 Q.K^T variant (bf16 inputs): permute_kv writes the key tiles as e4m3
// codes with one scale per 64-key sub-tile, quant_centroids does the same per
// 64 key centroids, and attn_fwd quantizes each query row in its prologue; S^T
// = K Q^T then runs on v_mfma_scale_f32_32x32x64_f8f6f4 and the tile's logit
// scale becomes scale * s_q * s_k. P.V and everything after it are as in the
// bf16 path.
// fp32 path: the same computation on VALU, one thread per query.
#include <type_traits>

#include "fp8.h"
#include "kernels.h"
#include "mfma.h"

namespace ca {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazy = 8.0f;   // log2 headroom before the running maximum moves

// Token indices come from caller-supplied permutations: out-of-range values
// read row 0 instead of faulting (the result is then meaningless).
CA_DEV int clamp_tok(int t, int N) { return (unsigned)t < (unsigned)N ? t : 0; }

// Storage slot of key k (0..15) inside a 16-key group of a transposed V tile:
// the middle two quads are swapped so that the 8 keys a lane contributes to
// the P.V contraction are contiguous.
CA_HD int vslot(int k) {
  const int q = (k >> 2) & 3;
  const int qs = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (k & ~15) | (qs << 2) | (k & 3);
}

// ----------------------------------------------------------------------------
// Cluster-major K / transposed V tiles and centroids (bf16 path)
// ----------------------------------------------------------------------------

template <int D, bool FP8>
__global__ __launch_bounds__(256) void permute_kv(AttnArgs a) {
  constexpr int RB = 64;                    // rows per LDS block (= one key sub-tile)
  __shared__ __attribute__((aligned(16))) uint16_t skr[RB][D + 8];
  __shared__ __attribute__((aligned(16))) uint16_t sv[RB][D + 8];
  __shared__ float sk[256 / D][D], sm[256 / D][D];
  __shared__ uint32_t samax[4];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int c = a.c, nc = a.nc, ncp = attn_ncp(nc);
  const int tid = threadIdx.x;
  if (j >= nc) {
    // centroid padding up to a whole sub-tile: zero vectors with ln n = -inf
    for (int d = tid; d < D; d += 256) {
      a.kbar_hi[((int64_t)bh * ncp + j) * D + d] = 0;
      a.vbar_t[(((int64_t)bh * (ncp / 64) + j / 64) * D + d) * 64 + vslot(j % 64)] = 0;
    }
    if (tid == 0) a.logn[(int64_t)bh * ncp + j] = kNegInf;
    return;
  }
  const int nj = min(c, a.N - j * c);
  const int32_t* perm = a.perm_k ? a.perm_k + (int64_t)bh * a.N + (int64_t)j * c : nullptr;
  const uint16_t* K = (const uint16_t*)a.K + (int64_t)(bh / a.kvg) * a.N * D;
  const uint16_t* V = (const uint16_t*)a.V + (int64_t)(bh / a.kvg) * a.N * D;
  uint16_t* kc = FP8 ? nullptr : a.kc + ((int64_t)bh * nc + j) * c * D;
  uint8_t* kc8 = FP8 ? a.kc8 + ((int64_t)bh * nc + j) * c * D : nullptr;
  uint16_t* vt = a.vt + ((int64_t)bh * nc + j) * (int64_t)D * c;

  // Blocks of 64 rows: the K and V chunks of block b + 1 are loaded while
  // block b is summed and transposed out of LDS. K rows go to kc straight from
  // registers (zero padded past the cluster's end); with FP8 they go out as
  // codes once the block's largest magnitude is known.
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int LPT = RB * CPR / 256;       // chunks per thread and block
  constexpr int G = 256 / D;
  const int d = tid % D, grp = tid / D;
  const int nb = c / RB;
  u32x4_t kr[LPT], vr[LPT];
  auto load = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = i * 256 + tid, r = b * RB + e / CPR, g = e % CPR;
      kr[i] = vr[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (r < nj) {
        const int tok = perm ? clamp_tok(perm[r], a.N) : j * c + r;
        kr[i] = *reinterpret_cast<const u32x4_t*>(K + (int64_t)tok * D + 8 * g);
        vr[i] = *reinterpret_cast<const u32x4_t*>(V + (int64_t)tok * D + 8 * g);
      }
    }
  };
  // centroid sums in row order: thread (grp, d) sums rows grp, grp + G, ...
  float ksum = 0.0f, vsum = 0.0f;
  load(0);
  for (int b = 0; b < nb; ++b) {
    if (b > 0) __syncthreads();   // the previous block's LDS reads are done
    uint32_t am = 0;              // FP8: largest |k| bits of this thread's chunks
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = i * 256 + tid, r = e / CPR, g = e % CPR;
      *reinterpret_cast<u32x4_t*>(&skr[r][8 * g]) = kr[i];
      *reinterpret_cast<u32x4_t*>(&sv[r][8 * g]) = vr[i];
      if constexpr (FP8) am = amax_bits_bf16x8(kr[i], am);
      else *reinterpret_cast<u32x4_t*>(kc + (int64_t)(b * RB + r) * D + 8 * g) = kr[i];
    }
    if constexpr (FP8) {
      const float wm = wave_max(bf16_to_f32((uint16_t)am));
      if ((tid & 63) == 0) samax[tid >> 6] = __float_as_uint(wm);
    } else {
      if (b + 1 < nb) load(b + 1);
    }
    __syncthreads();
    if constexpr (FP8) {
      const float amax = fmaxf(fmaxf(__uint_as_float(samax[0]), __uint_as_float(samax[1])),
                               fmaxf(__uint_as_float(samax[2]), __uint_as_float(samax[3])));
      const float inv = e4m3_inv(amax);
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int e = i * 256 + tid, r = e / CPR, g = e % CPR;
        *reinterpret_cast<u32x2_t*>(kc8 + (int64_t)(b * RB + r) * D + 8 * g) = e4m3_pack_bf16x8(kr[i], inv);
      }
      if (tid == 0) a.kscale[((int64_t)bh * nc + j) * (c / RB) + b] = e4m3_scale(amax);
      if (b + 1 < nb) load(b + 1);
    }
    for (int r = grp; r < RB && b * RB + r < nj; r += G) {
      ksum += bf16_to_f32(skr[r][d]);
      vsum += bf16_to_f32(sv[r][d]);
    }
    // V written transposed [D][64] per block: each thread writes 8
    // consecutive storage slots of one dim
    for (int e = tid; e < D * (RB / 8); e += 256) {
      const int dd = e / (RB / 8), s8 = e % (RB / 8);
      uint16_t vals[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // storage slot s8*8+q holds key vslot^-1(slot); vslot is an involution
        const int key = vslot(s8 * 8 + q);
        vals[q] = sv[key][dd];
      }
      u32x4_t pk;
      pk.x = vals[0] | ((uint32_t)vals[1] << 16);
      pk.y = vals[2] | ((uint32_t)vals[3] << 16);
      pk.z = vals[4] | ((uint32_t)vals[5] << 16);
      pk.w = vals[6] | ((uint32_t)vals[7] << 16);
      *reinterpret_cast<u32x4_t*>(vt + (int64_t)b * D * RB + dd * RB + s8 * 8) = pk;
    }
  }
  sk[grp][d] = ksum;
  sm[grp][d] = vsum;
  __syncthreads();
  if (grp == 0) {
    float ks = 0.0f, vs = 0.0f;
#pragma unroll
    for (int q = 0; q < G; ++q) { ks += sk[q][d]; vs += sm[q][d]; }
    const float inv = 1.0f / (float)nj;
    const float kb = ks * inv, vb = vs * inv;
    a.kbar_hi[((int64_t)bh * ncp + j) * D + d] = f32_to_bf16(kb);
    a.vbar_t[(((int64_t)bh * (ncp / 64) + j / 64) * D + d) * 64 + vslot(j % 64)] = f32_to_bf16(vb);
    if (d == 0) a.logn[(int64_t)bh * ncp + j] = logf((float)nj);
  }
}

// FP8: key centroids (bf16, written by permute_kv) as e4m3 codes with one
// scale per 64 consecutive centroids; one workgroup per 64 centroids.
template <int D>
__global__ __launch_bounds__(256) void quant_centroids(AttnArgs a) {
  constexpr int RB = 64, CPR = D / 8, LPT = RB * CPR / 256;
  __shared__ uint32_t samax[4];
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int ncp = attn_ncp(a.nc);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.kbar_hi + ((int64_t)bh * ncp + blk * RB) * D);
  uint8_t* dst = a.kbar8 + ((int64_t)bh * ncp + blk * RB) * D;
  u32x4_t v[LPT];
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    v[i] = src[i * 256 + tid];
    am = amax_bits_bf16x8(v[i], am);
  }
  const float wm = wave_max(bf16_to_f32((uint16_t)am));
  if ((tid & 63) == 0) samax[tid >> 6] = __float_as_uint(wm);
  __syncthreads();
  const float amax = fmaxf(fmaxf(__uint_as_float(samax[0]), __uint_as_float(samax[1])),
                           fmaxf(__uint_as_float(samax[2]), __uint_as_float(samax[3])));
  const float inv = e4m3_inv(amax);
#pragma unroll
  for (int i = 0; i < LPT; ++i)
    *reinterpret_cast<u32x2_t*>(dst + (int64_t)(i * 256 + tid) * 8) = e4m3_pack_bf16x8(v[i], inv);
  if (tid == 0) a.kbscale[(int64_t)bh * (ncp / RB) + blk] = e4m3_scale(amax);
}

// ----------------------------------------------------------------------------
// Attention (bf16 MFMA)
// ----------------------------------------------------------------------------

// Key/value sub-tiles of 64 keys are staged in LDS, double buffered: K rows
// (64 x D bf16) and V^T rows (D x 64 bf16), each row padded by 16 bytes so
// that the 16 lanes an LDS cycle serves (16 consecutive rows at one 16-byte
// chunk) fall on distinct banks and every operand read is a per-lane base
// plus a compile-time offset.
// With FP8 keys a K row is D bytes (+16 of padding, which again puts the 16
// rows an LDS cycle serves on distinct banks).
template <int D, bool FP8 = false>
struct AttnTile {
  static constexpr int KT = 64;                           // keys per sub-tile
  static constexpr int KE = FP8 ? 1 : 2;                  // bytes per key element
  static constexpr int KP = D * KE + 16;                  // K row pitch (bytes)
  static constexpr int VP = KT * 2 + 16;                  // V^T row pitch (bytes)
  static constexpr int K_BYTES = KT * KP;
  static constexpr int V_BYTES = D * VP;
  static constexpr int BYTES = K_BYTES + V_BYTES;         // one buffer
  static constexpr int K_CHUNKS = D * KE / 16;            // 16-byte chunks per K row
  static constexpr int V_CHUNKS = KT / 8;                 // 16-byte chunks per V^T row
  static constexpr int K_LOADS = KT * K_CHUNKS;           // 16-byte loads per sub-tile
  static constexpr int V_LOADS = D * V_CHUNKS;
};

// Workgroup order: consecutive logical workgroups (adjacent query clusters of
// one head, which select overlapping key clusters) are kept on one XCD, whose
// L2 then serves their shared key/value tiles. Hardware hands workgroup b to
// XCD b % 8.
CA_DEV int xcd_logical(int b, int G) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = G >> 3, rem = G & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// KSPL = 2 (64-query clusters): the workgroup has two waves per 32 queries,
// each taking one 32-key half of every sub-tile with its own running maximum,
// sum and accumulators, merged through LDS at the end. This keeps four waves
// (and the per-thread share of the tile loads) of a 128-query workgroup.
template <int D, int CQ, int CK, bool DENSE, bool FP8, int KSPL>
__global__ __launch_bounds__(2 * CQ * KSPL) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd(AttnArgs a) {
  using TL = AttnTile<D, FP8>;
  constexpr int NT = 2 * CQ * KSPL;    // threads: CQ/32 query groups x KSPL key halves
  constexpr int NKB = 2 / KSPL;        // 32-key blocks of a sub-tile per wave
  constexpr int KS = D / 16;           // k-steps over the head dim
  constexpr int NB = D / 32;           // 32-row blocks of O^T
  constexpr int SUB = CK / TL::KT;     // sub-tiles per key cluster
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* sSel = reinterpret_cast<uint32_t*>(smem + 2 * TL::BYTES);

  const int G = gridDim.x * gridDim.y;
  const int lg = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, G);
  const int nc = a.nc, nqc = a.nqc, N = a.N;   // key clusters, query clusters
  const int qa = lg % nqc, bh = lg / nqc;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, r = l & 31;
  const int qg = w % (CQ / 32);                                             // query group
  const int kh = KSPL == 1 ? 0 : __builtin_amdgcn_readfirstlane(w / (CQ / 32));   // key half
  const int qpos = qa * CQ + qg * 32 + r;
  const bool qvalid = qpos < N;
  const int qtok =
      qvalid ? (DENSE || !a.perm_q ? qpos : clamp_tok(a.perm_q[(int64_t)bh * N + qpos], N)) : 0;
  const uint16_t* Qh = (const uint16_t*)a.Q + (int64_t)bh * N * D;

  // Query operand. bf16: step s of the contraction covers dims 16s..16s+15,
  // lane half h supplying 8 of them. FP8: step s covers dims 64s..64s+63,
  // lane half h supplying the 32 dims from 64s + 32h as e4m3 codes of the
  // row quantized with its own scale sq (the halves combine their maxima).
  constexpr int KS8 = D / 64;
  bf16x8_t qf[FP8 ? 1 : KS];
  i32x8_t qf8[FP8 ? KS8 : 1];
  float sq = 1.0f;
  if constexpr (FP8) {
    u32x4_t v[KS8][4];
    uint32_t am = 0;
#pragma unroll
    for (int s = 0; s < KS8; ++s)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        v[s][c4] = u32x4_t{0u, 0u, 0u, 0u};
        if (qvalid) v[s][c4] = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)qtok * D + s * 64 + h * 32 + c4 * 8);
        am = amax_bits_bf16x8(v[s][c4], am);
      }
    const float amax = max_halves(bf16_to_f32((uint16_t)am));
    const float inv = e4m3_inv(amax);
    sq = e4m3_scale(amax);
#pragma unroll
    for (int s = 0; s < KS8; ++s)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const u32x2_t w = e4m3_pack_bf16x8(v[s][c4], inv);
        qf8[s][2 * c4] = (int)w.x;
        qf8[s][2 * c4 + 1] = (int)w.y;
      }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)qtok * D + s * 16 + h * 8);
      qf[s] = as_bf16x8(v);
    }
  }
  floatx16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = zero16();
  float m = kNegInf, lsum = 0.0f;
  const float sl2 = a.scale * kLog2e;

  const int nsel = DENSE ? nc
                  : (a.nsel ? min(max(a.nsel[(int64_t)bh * nqc + qa], 0), a.topk) : a.topk);
  const int32_t* blk = DENSE ? nullptr : a.blocks + ((int64_t)bh * nqc + qa) * a.topk;
  // Token sub-tiles of the selected clusters come first; with compensation the
  // centroids follow as ncp / 64 more sub-tiles of 64 (kbar rows as keys,
  // vbar as values) whose logits get + ln n_c, or -inf for a selected or
  // padding cluster, in the same running maximum and sum.
  const int Tm = nsel * SUB;
  const int ncp = attn_ncp(nc);
  const bool comp = !DENSE && a.compensate;
  const int T = Tm + (comp ? ncp / TL::KT : 0);
  if (comp) {
    for (int e = tid; e < ncp / 32; e += NT) sSel[e] = 0u;
    __syncthreads();
    for (int e = tid; e < nsel; e += NT) {
      const int j = blk[e];
      if (j >= 0 && j < nc) atomicOr(&sSel[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }

  // cluster of token sub-tile t (out-of-range block entries are skipped)
  auto tile_cluster = [&](int t) -> int {
    const int j = DENSE ? t / SUB : blk[t / SUB];
    return (j >= 0 && j < nc) ? j : -1;
  };
  // stage: 16-byte global loads into registers, then into an LDS buffer
  // (with FP8 and D = 64 a K sub-tile is 256 loads: fewer than 512 threads)
  constexpr int KLPT = (TL::K_LOADS + NT - 1) / NT, VLPT = TL::V_LOADS / NT;
  constexpr bool K_ALL = TL::K_LOADS % NT == 0;
  static_assert(TL::V_LOADS % NT == 0, "V sub-tile loads must divide evenly");
  u32x4_t kst[KLPT], vst[VLPT];
  float ksc_cur = 1.0f, ksc_nxt = 1.0f;   // FP8: key scale of the current / next sub-tile
  // Every sub-tile is contiguous in HBM (K rows [64][D], V^T rows [D][64],
  // token and centroid tiles alike), so each thread's 16-byte chunks sit at
  // fixed offsets from a per-tile base.
  auto fetch = [&](int t) {
    const u32x4_t* ks;
    const u32x4_t* vs;
    if (t < Tm) {
      int j = tile_cluster(t);
      if (j < 0) j = 0;   // any valid tile; its results are not used
      const int part = t % SUB;
      const int64_t row = ((int64_t)bh * nc + j) * CK + part * TL::KT;
      if constexpr (FP8) {
        ks = reinterpret_cast<const u32x4_t*>(a.kc8 + row * D);
        ksc_nxt = a.kscale[((int64_t)bh * nc + j) * SUB + part];
      } else {
        ks = reinterpret_cast<const u32x4_t*>(a.kc + row * D);
      }
      vs = reinterpret_cast<const u32x4_t*>(a.vt + (((int64_t)bh * nc + j) * SUB + part) * (int64_t)D * TL::KT);
    } else {
      const int ct = t - Tm;
      if constexpr (FP8) {
        ks = reinterpret_cast<const u32x4_t*>(a.kbar8 + ((int64_t)bh * ncp + ct * TL::KT) * D);
        ksc_nxt = a.kbscale[(int64_t)bh * (ncp / TL::KT) + ct];
      } else {
        ks = reinterpret_cast<const u32x4_t*>(a.kbar_hi + ((int64_t)bh * ncp + ct * TL::KT) * D);
      }
      vs = reinterpret_cast<const u32x4_t*>(a.vbar_t + ((int64_t)bh * (ncp / TL::KT) + ct) * D * TL::KT);
    }
#pragma unroll
    for (int i = 0; i < KLPT; ++i)
      if (K_ALL || i * NT + tid < TL::K_LOADS) kst[i] = ks[i * NT + tid];
#pragma unroll
    for (int i = 0; i < VLPT; ++i) vst[i] = vs[i * NT + tid];
  };
  auto store = [&](int buf) {
    unsigned char* base = smem + buf * TL::BYTES;
#pragma unroll
    for (int i = 0; i < KLPT; ++i) {
      const int e = i * NT + tid;
      if (K_ALL || e < TL::K_LOADS)
        *reinterpret_cast<u32x4_t*>(base + (e / TL::K_CHUNKS) * TL::KP + (e % TL::K_CHUNKS) * 16) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < VLPT; ++i) {
      const int e = i * NT + tid;
      *reinterpret_cast<u32x4_t*>(base + TL::K_BYTES + (e / TL::V_CHUNKS) * TL::VP +
                                  (e % TL::V_CHUNKS) * 16) = vst[i];
    }
  };
  // per-lane LDS read bases: K row r, chunk h (FP8: 32-byte chunk h); V^T
  // row r, chunk h
  const int kread = r * TL::KP + h * (FP8 ? 32 : 16);
  const int vread = TL::K_BYTES + r * TL::VP + h * 16;
  const float* logn = a.logn + (int64_t)bh * ncp;

  if (T > 0) {
    fetch(0);
    store(0);
    ksc_cur = ksc_nxt;
  }
  __syncthreads();
  // Sub-tiles that need no masking (full token tiles) run in loops of their
  // own; the sub-tiles of the short last cluster, wherever the selection
  // holds it, and the centroid tiles run in loops with the masking code.
  int rpos = -1;   // position of the short cluster in the selection, if any
  if (N % CK != 0) {
    if (DENSE) {
      rpos = nc - 1;
    } else {
      int mine = -1;   // entries are distinct: at most one lane finds it
      for (int e = l; e < nsel; e += 64)
        if (blk[e] == nc - 1) mine = e;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mine = max(mine, __shfl_xor(mine, o, 64));
      rpos = __builtin_amdgcn_readfirstlane(mine);
    }
  }
  auto step = [&](int t, auto special_tag) __attribute__((always_inline)) {
    constexpr bool SPECIAL = decltype(special_tag)::value;
    if (t + 1 < T) fetch(t + 1);
    const bool cen = SPECIAL && t >= Tm;
    const int j = cen ? 0 : tile_cluster(t);
    if (j >= 0) {
      const unsigned char* buf = smem + (t & 1) * TL::BYTES;
      const int nvalid = cen ? TL::KT : min(CK, N - j * CK) - (t % SUB) * TL::KT;
      // two independent accumulation chains interleaved: the two 32-key
      // blocks, or (KSPL = 2) the even and odd k-steps of the wave's block,
      // added afterwards. Product i covers key block kbg(i) and k-step s(i).
      floatx16_t sacc[2] = {zero16(), zero16()};
      auto kblk = [&](int i) { return KSPL == 1 ? (i & 1) : kh; };
      if constexpr (FP8) {
        // NKB x KS8 products of 32 keys x 64 dims; every operand read issued first
        constexpr int NQ = NKB * KS8;
        i32x8_t kf[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i)
          kf[i] = *reinterpret_cast<const i32x8_t*>(buf + kread + kblk(i) * 32 * TL::KP + (i / NKB) * 64);
#pragma unroll
        for (int i = 0; i < NQ; ++i) sacc[i & 1] = mfma32_fp8(kf[i], qf8[i / NKB], sacc[i & 1]);
      } else {
        // operand reads issued PF ahead of their products (ring of PF
        // registers); the schedule is pinned by scheduling barriers
        constexpr int NQ = NKB * KS, PF = 4;
        bf16x8_t ring[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i)
          ring[i] = *reinterpret_cast<const bf16x8_t*>(buf + kread + kblk(i) * 32 * TL::KP + (i / NKB) * 32);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          __builtin_amdgcn_sched_barrier(0);
          sacc[i & 1] = mfma32(ring[i % PF], qf[i / NKB], sacc[i & 1]);
          if (i + PF < NQ) {
            const int j = i + PF;
            ring[i % PF] = *reinterpret_cast<const bf16x8_t*>(buf + kread + kblk(j) * 32 * TL::KP + (j / NKB) * 32);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (KSPL == 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[0][i] += sacc[1][i];
      }
      // the exponent below is fma(score, scl, -m): token tiles keep raw q.k
      // (scl = scale log2 e, times s_q s_k with FP8), centroid tiles are
      // turned into log2 units here
      // (floored at the smallest normal fp32 so that a zero query or key
      // block gives logits 0, and masked keys stay at -inf)
      float scl = FP8 ? fmaxf(sl2 * sq * ksc_cur, __FLT_MIN__) : sl2;
      if (SPECIAL && cen) {
        const float sc = scl;
        scl = 1.0f;
        const int c0 = (t - Tm) * TL::KT;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k0 = c0 + (KSPL == 1 ? kb : kh) * 32 + 8 * q + 4 * h;
            const floatx4_t ln = *reinterpret_cast<const floatx4_t*>(logn + k0);
            const uint32_t selw = sSel[k0 >> 5];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool excluded = !((selw >> ((k0 + e) & 31)) & 1u);
              const float bias = excluded ? ln[e] * kLog2e : kNegInf;
              sacc[kb][4 * q + e] = fmaf(sacc[kb][4 * q + e], sc, bias);
            }
          }
      } else if (SPECIAL && nvalid < TL::KT) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool out = (KSPL == 1 ? kb : kh) * 32 + c_row(i, h) >= nvalid;
            sacc[kb][i] = out ? kNegInf : sacc[kb][i];
          }
      }
      // online softmax with a lazily updated running maximum: m only moves
      // (and the accumulators are rescaled) when the tile's maximum exceeds
      // it by more than 2^8, so P <= 256 (exact after the final division by
      // l, which uses the same m)
      float bm = kNegInf;
#pragma unroll
      for (int i = 0; i < 16 * NKB; ++i) bm = fmaxf(bm, sacc[i >> 4][i & 15]);
      bm = max_halves(bm) * scl;
      const bool grow = bm > m + kLazy;
      if (__ballot(grow)) [[unlikely]] {
        const float mn = grow ? bm : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
        lsum *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][i] *= alpha;
        m = mn;
      }
      const float nm = m == kNegInf ? 0.0f : -m;   // nothing valid yet: P = 0
      float tv[16 * NKB];
#pragma unroll
      for (int i = 0; i < 16 * NKB; ++i) tv[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 4][i & 15], scl, nm));
      // P enters the P.V product as bf16; the denominator sums the same
      // rounded values, so the output stays a convex combination of values
      bf16x8_t pk[2 * NKB];
      float ps = 0.0f;
#pragma unroll
      for (int q = 0; q < 2 * NKB; ++q) {
        const u32x4_t u = pack8(tv + 8 * q);
        ps = sum_bf16x8(u, ps);
        pk[q] = as_bf16x8(u);
      }
      lsum += ps;   // this lane's keys; the halves are added at the end
      {
        // keys 16q .. 16q+15 of the sub-tile: V^T chunk 2q + h (q counted
        // from the wave's key half); reads issued PF ahead of their products
        constexpr int NV = 2 * NKB * NB, PF = 4;
        const int vq0 = 2 * kh;
        bf16x8_t ring[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i)
          ring[i] = *reinterpret_cast<const bf16x8_t*>(buf + vread + (i % NB) * 32 * TL::VP + (vq0 + i / NB) * 32);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          __builtin_amdgcn_sched_barrier(0);
          const int nb = i % NB, q = i / NB;
          acc[nb] = mfma32(ring[i % PF], pk[q], acc[nb]);
          if (i + PF < NV) {
            const int j = i + PF;
            ring[i % PF] = *reinterpret_cast<const bf16x8_t*>(buf + vread + (j % NB) * 32 * TL::VP + (vq0 + j / NB) * 32);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t + 1 < T) store((t + 1) & 1);
    ksc_cur = ksc_nxt;
    __syncthreads();
  };
  auto run = [&](int t0, int t1, auto special_tag) __attribute__((always_inline)) {
#pragma unroll 1
    for (int t = t0; t < t1; ++t) step(t, special_tag);
  };
  if (rpos < 0) {
    run(0, Tm, std::false_type{});
  } else {
    run(0, rpos * SUB, std::false_type{});
    run(rpos * SUB, rpos * SUB + SUB, std::true_type{});
    run(rpos * SUB + SUB, Tm, std::false_type{});
  }
  run(Tm, T, std::true_type{});

  lsum = sum_halves(lsum);
  if constexpr (KSPL == 2) {
    // merge the key halves: the second wave of each query group leaves its
    // maximum, sum and accumulators in LDS (the tile buffers are free after
    // the last barrier), the first rescales both to the larger maximum
    constexpr int XE = 16 * NB + 2;   // floats per lane
    static_assert((CQ / 32) * XE * 64 * 4 <= 2 * TL::BYTES, "exchange fits the tile buffers");
    float* xch = reinterpret_cast<float*>(smem) + (size_t)qg * XE * 64 + l;
    if (kh == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(nb * 16 + i) * 64] = acc[nb][i];
      xch[16 * NB * 64] = m;
      xch[(16 * NB + 1) * 64] = lsum;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xch[16 * NB * 64], l1 = xch[(16 * NB + 1) * 64];
    const float mn = fmaxf(m, m1);
    const float a0 = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    const float a1 = m1 == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m1 - mn);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = fmaf(acc[nb][i], a0, xch[(nb * 16 + i) * 64] * a1);
    lsum = fmaf(lsum, a0, l1 * a1);
    m = mn;
  }
  if (!qvalid) return;
  const float inv = 1.0f / lsum;
  uint16_t* Oh = (uint16_t*)a.O + ((int64_t)bh * N + qtok) * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = nb * 32 + 8 * g + 4 * h;
      u32x2_t v;
      v.x = pack_bf16x2(acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv);
      v.y = pack_bf16x2(acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv);
      *reinterpret_cast<u32x2_t*>(Oh + d0) = v;
    }
  }
  if (a.lse && h == 0) a.lse[(int64_t)bh * N + qtok] = (m + log2f(lsum)) * kLn2;
}

template <int D, bool FP8>
constexpr size_t attn_smem() {
  return 2 * (size_t)AttnTile<D, FP8>::BYTES + 8192 / 8 + 64;   // two buffers, selection bits
}

// ----------------------------------------------------------------------------
// fp32 path
// ----------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void centroids_kv_f32(AttnArgs a) {
  const int j = blockIdx.x, bh = blockIdx.y;
  const int ncp = attn_ncp(a.nc);
  const int d = threadIdx.x;
  if (d >= D) return;
  float* kb = a.kbar32 + ((int64_t)bh * ncp + j) * D;
  float* vb = a.vbar32 + ((int64_t)bh * ncp + j) * D;
  if (j >= a.nc) {
    kb[d] = 0.0f; vb[d] = 0.0f;
    if (d == 0) a.logn[(int64_t)bh * ncp + j] = kNegInf;
    return;
  }
  const int nj = min(a.c, a.N - j * a.c);
  const int32_t* perm = a.perm_k + (int64_t)bh * a.N + (int64_t)j * a.c;
  const float* K = (const float*)a.K + (int64_t)(bh / a.kvg) * a.N * D;
  const float* V = (const float*)a.V + (int64_t)(bh / a.kvg) * a.N * D;
  float ks = 0.0f, vs = 0.0f;
  for (int r = 0; r < nj; ++r) {
    const int tok = clamp_tok(perm[r], a.N);
    ks += K[(int64_t)tok * D + d];
    vs += V[(int64_t)tok * D + d];
  }
  kb[d] = ks / (float)nj;
  vb[d] = vs / (float)nj;
  if (d == 0) a.logn[(int64_t)bh * ncp + j] = logf((float)nj);
}

template <int D, bool DENSE>
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
  __shared__ float skv[2][32][D];
  __shared__ uint32_t sSel[8192 / 32];
  const int qa = blockIdx.x, bh = blockIdx.y;
  const int N = a.N, nc = a.nc, c = a.c, cq = a.cq, nqc = a.nqc;
  const int tid = threadIdx.x;
  const int qpos = qa * 256 + tid;                   // DENSE: 256 queries per block
  int qtok = 0;
  bool qvalid;
  if (DENSE) {
    qvalid = qpos < N;
    qtok = qpos;
  } else {
    const int nq = min(cq, N - qa * cq);
    qvalid = tid < nq;
    if (qvalid) qtok = clamp_tok(a.perm_q[(int64_t)bh * N + qa * cq + tid], N);
  }
  const float* Qh = (const float*)a.Q + (int64_t)bh * N * D;
  const float* Kh = (const float*)a.K + (int64_t)(bh / a.kvg) * N * D;
  const float* Vh = (const float*)a.V + (int64_t)(bh / a.kvg) * N * D;
  float q[D], o[D];
  for (int d = 0; d < D; ++d) { q[d] = qvalid ? Qh[(int64_t)qtok * D + d] : 0.0f; o[d] = 0.0f; }
  float m = kNegInf, lsum = 0.0f;
  auto absorb = [&](float logit, const float* v) {
    const float mn = fmaxf(m, logit);
    const float alpha = __expf(m - mn);
    const float p = __expf(logit - mn);
    lsum = lsum * alpha + p;
    for (int d = 0; d < D; ++d) o[d] = o[d] * alpha + p * v[d];
    m = mn;
  };
  // key tokens, 32 at a time through LDS
  const int nsel = DENSE ? 1
                  : (a.nsel ? min(max(a.nsel[(int64_t)bh * nqc + qa], 0), a.topk) : a.topk);
  for (int bi = 0; bi < nsel; ++bi) {
    const int j = DENSE ? 0 : a.blocks[((int64_t)bh * nqc + qa) * a.topk + bi];
    if (j < 0 || j >= nc) continue;
    const int kbeg = DENSE ? 0 : j * c;
    const int kcnt = DENSE ? N : min(c, N - j * c);
    for (int k0 = 0; k0 < kcnt; k0 += 32) {
      __syncthreads();
      for (int e = tid; e < 32 * D; e += 256) {
        const int rr = e / D, d = e % D;
        if (k0 + rr < kcnt) {
          const int pos = kbeg + k0 + rr;
          const int tok = DENSE ? pos : clamp_tok(a.perm_k[(int64_t)bh * N + pos], N);
          skv[0][rr][d] = Kh[(int64_t)tok * D + d];
          skv[1][rr][d] = Vh[(int64_t)tok * D + d];
        }
      }
      __syncthreads();
      const int kn = min(32, kcnt - k0);
      for (int rr = 0; rr < kn; ++rr) {
        float s = 0.0f;
        for (int d = 0; d < D; ++d) s += q[d] * skv[0][rr][d];
        absorb(s * a.scale, skv[1][rr]);
      }
    }
  }
  if (!DENSE && a.compensate) {
    const int ncp = attn_ncp(nc);
    __syncthreads();
    for (int e = tid; e < ncp / 32; e += 256) sSel[e] = 0u;
    __syncthreads();
    for (int e = tid; e < nsel; e += 256) {
      const int j = a.blocks[((int64_t)bh * nqc + qa) * a.topk + e];
      if (j >= 0 && j < nc) atomicOr(&sSel[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    for (int j = 0; j < nc; ++j) {
      if ((sSel[j >> 5] >> (j & 31)) & 1u) continue;
      const float* kb = a.kbar32 + ((int64_t)bh * ncp + j) * D;
      const float* vb = a.vbar32 + ((int64_t)bh * ncp + j) * D;
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s += q[d] * kb[d];
      absorb(s * a.scale + a.logn[(int64_t)bh * ncp + j], vb);
    }
  }
  if (!qvalid) return;
  float* Oh = (float*)a.O + ((int64_t)bh * N + qtok) * D;
  const float inv = 1.0f / lsum;
  for (int d = 0; d < D; ++d) Oh[d] = o[d] * inv;
  if (a.lse) a.lse[(int64_t)bh * N + qtok] = m + logf(lsum);
}

template <int D, int CQ, int CK, bool DENSE, bool FP8>
void launch_mfma(const AttnArgs& a, hipStream_t st) {
  constexpr int KSPL = CQ == 64 ? 2 : 1;
  const size_t sm = attn_smem<D, FP8>();
  static bool attr_set = false;   // raise the dynamic-LDS limit once per instantiation
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd<D, CQ, CK, DENSE, FP8, KSPL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    attr_set = true;
  }
  dim3 g(a.nqc, a.BH);
  if (a.ev_start) (void)hipEventRecord(a.ev_start, st);
  attn_fwd<D, CQ, CK, DENSE, FP8, KSPL><<<g, 2 * CQ * KSPL, sm, st>>>(a);
  if (a.ev_stop) (void)hipEventRecord(a.ev_stop, st);
}

template <int D, bool FP8>
void launch_tiles(const AttnArgs& a, bool dense, hipStream_t st) {
  dim3 gp(attn_ncp(a.nc), a.BH);
  permute_kv<D, FP8><<<gp, 256, 0, st>>>(a);
  if (FP8 && !dense && a.compensate) {
    dim3 gq(attn_ncp(a.nc) / 64, a.BH);
    quant_centroids<D><<<gq, 256, 0, st>>>(a);
  }
  if (dense) {
    launch_mfma<D, 128, 128, true, FP8>(a, st);
    return;
  }
  // (query, key) cluster sizes: equal, or the key clusters larger
  switch (a.cq * 1000 + a.c) {
    case 64064: launch_mfma<D, 64, 64, false, FP8>(a, st); break;
    case 64128: launch_mfma<D, 64, 128, false, FP8>(a, st); break;
    case 64256: launch_mfma<D, 64, 256, false, FP8>(a, st); break;
    case 128128: launch_mfma<D, 128, 128, false, FP8>(a, st); break;
    case 128256: launch_mfma<D, 128, 256, false, FP8>(a, st); break;
    default: launch_mfma<D, 256, 256, false, FP8>(a, st); break;
  }
}

template <int D>
void launch_bf16(const AttnArgs& a, bool dense, hipStream_t st) {
  if (a.dtype == 2) launch_tiles<D, true>(a, dense, st);
  else launch_tiles<D, false>(a, dense, st);
}

template <int D>
void launch_f32(const AttnArgs& a, bool dense, hipStream_t st) {
  if (dense) {
    dim3 g((a.N + 255) / 256, a.BH);
    if (a.ev_start) (void)hipEventRecord(a.ev_start, st);
    attn_f32<D, true><<<g, 256, 0, st>>>(a);
    if (a.ev_stop) (void)hipEventRecord(a.ev_stop, st);
    return;
  }
  dim3 gc(attn_ncp(a.nc), a.BH);
  centroids_kv_f32<D><<<gc, 256, 0, st>>>(a);
  dim3 g(a.nqc, a.BH);
  if (a.ev_start) (void)hipEventRecord(a.ev_start, st);
  attn_f32<D, false><<<g, 256, 0, st>>>(a);
  if (a.ev_stop) (void)hipEventRecord(a.ev_stop, st);
}

}  // namespace

void launch_attend(const AttnArgs& a, hipStream_t st) {
  if (a.dtype != 1) {
    if (a.D == 64) launch_bf16<64>(a, false, st); else launch_bf16<128>(a, false, st);
  } else {
    if (a.D == 64) launch_f32<64>(a, false, st); else launch_f32<128>(a, false, st);
  }
}

void launch_dense(const AttnArgs& a, hipStream_t st) {
  if (a.dtype != 1) {
    if (a.D == 64) launch_bf16<64>(a, true, st); else launch_bf16<128>(a, true, st);
  } else {
    if (a.D == 64) launch_f32<64>(a, true, st); else launch_f32<128>(a, true, st);
  }
}

}  // namespace ca
