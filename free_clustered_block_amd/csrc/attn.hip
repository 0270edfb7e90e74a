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
// FP8 Q.K^T and P.V variant: in addition, the values enter P.V as e4m3
// codes with a power-of-two scale per head dimension and 32 keys (the OCP
// microscaling block scale, applied by v_mfma_scale_f32_32x32x64_f8f6f4 to
// its A operand), written by permute_kv (quant_vcentroids for the value
// centroids), and the attention weights are rounded to e4m3 (they are at
// most 2^8 by the lazy running maximum, inside the format's range) before
// the product; the softmax denominator sums the fp32 weights.
// fp32 path: the same computation on VALU, one thread per query.
#include <algorithm>
#include <type_traits>
#include <utility>

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

// FP8 value sub-tile (64 keys), in HBM and in LDS: D rows of 64 code bytes,
// then the scale bytes [2][32][4] (key block kb of 32 keys, dimension
// 32 nb + r at [kb][r][nb], byte = exponent + 127). Byte 32 h + 16 kb + j
// of a row holds key 32 kb + 16 h + j: the matrix core takes the 32 bytes
// of lane half h as its operand and scales bytes 16 kb .. 16 kb + 15 of both
// halves with the scale that lane half kb supplies, so each scale block is
// 32 consecutive keys; attn_fwd holds the weights in the same order.
template <int D>
constexpr int vt8_bytes() { return D * 64 + 256; }

// Codes and scale of dimension dd, key half hb of a 64-key block whose bf16
// values val(k) (k = key within the block) are given; dst is the sub-tile.
template <int D, typename F>
CA_DEV void write_vt8(uint8_t* dst, int dd, int hb, F val) {
  uint32_t am = 0;
#pragma unroll 8
  for (int k = 0; k < 32; ++k) am = max(am, (uint32_t)(val(32 * hb + k) & 0x7FFFu));
  const int ex = e8m0_exponent(bf16_to_f32((uint16_t)am));
  const float sc = ldexpf(1.0f, -ex);   // exact: a power of two
  uint32_t wv[8];   // keys 32 hb + 4 i + 0..3
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k0 = 32 * hb + 4 * i;
    wv[i] = e4m3_pack4_raw(bf16_to_f32(val(k0)) * sc, bf16_to_f32(val(k0 + 1)) * sc,
                           bf16_to_f32(val(k0 + 2)) * sc, bf16_to_f32(val(k0 + 3)) * sc);
  }
  // keys 32 hb + 16 h + j at byte 32 h + 16 hb + j
  *reinterpret_cast<u32x4_t*>(dst + dd * 64 + 16 * hb) = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
  *reinterpret_cast<u32x4_t*>(dst + dd * 64 + 32 + 16 * hb) = u32x4_t{wv[4], wv[5], wv[6], wv[7]};
  dst[D * 64 + (hb * 32 + (dd & 31)) * 4 + (dd >> 5)] = (uint8_t)(ex + 127);
}

// ----------------------------------------------------------------------------
// Cluster-major K / transposed V tiles and centroids (bf16 path)
// ----------------------------------------------------------------------------

template <int D, bool FP8, bool FP8PV>
__global__ __launch_bounds__(256) void permute_kv(AttnArgs a) {
  constexpr int RB = 64;                    // rows per LDS block (= one key sub-tile)
  __shared__ __attribute__((aligned(16))) uint16_t skr[RB][D + 8];
  __shared__ __attribute__((aligned(16))) uint16_t sv[RB][D + 8];
  __shared__ float sk[256 / D][D], sm[256 / D][D];
  __shared__ uint32_t samax[4];
  const int j = blockIdx.x, bh = blockIdx.y * (a.kshare > 1 ? a.kshare : 1);   // heads that build tiles
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
    if constexpr (FP8PV) {
      // FP8 values: thread (dim, key half) writes its 32 codes and scale
      uint8_t* vt8 = a.vt8 + (((int64_t)bh * nc + j) * (c / RB) + b) * vt8_bytes<D>();
      for (int e = tid; e < 2 * D; e += 256)
        write_vt8<D>(vt8, e % D, e / D, [&](int k) { return sv[k][e % D]; });
    }
    // V written transposed [D][64] per block: each thread writes 8
    // consecutive storage slots of one dim
    for (int e = tid; e < (FP8PV ? 0 : D * (RB / 8)); e += 256) {
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
  const int blk = blockIdx.x, bh = blockIdx.y * (a.kshare > 1 ? a.kshare : 1), tid = threadIdx.x;
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

// FP8 P.V: value centroids (bf16, written by permute_kv as transposed
// sub-tiles) as FP8 value sub-tiles; one workgroup per 64 centroids.
template <int D>
__global__ __launch_bounds__(256) void quant_vcentroids(AttnArgs a) {
  const int blk = blockIdx.x, bh = blockIdx.y * (a.kshare > 1 ? a.kshare : 1), tid = threadIdx.x;
  const int ncp = attn_ncp(a.nc);
  const uint16_t* src = a.vbar_t + ((int64_t)bh * (ncp / 64) + blk) * D * 64;
  uint8_t* dst = a.vbar8 + ((int64_t)bh * (ncp / 64) + blk) * vt8_bytes<D>();
  for (int e = tid; e < 2 * D; e += 256) {
    const int dd = e % D;
    write_vt8<D>(dst, dd, e / D, [&](int k) { return src[dd * 64 + vslot(k)]; });
  }
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
// With FP8 values a V^T row is 64 code bytes (+16 of padding: conflict-free
// 32-byte operand reads) and the sub-tile's 256 scale bytes follow the rows.
template <int D, bool FP8 = false, bool FP8PV = false>
struct AttnTile {
  static constexpr int KT = 64;                           // keys per sub-tile
  static constexpr int KE = FP8 ? 1 : 2;                  // bytes per key element
  static constexpr int KP = D * KE + 16;                  // K row pitch (bytes)
  static constexpr int VP = FP8PV ? KT + 16 : KT * 2 + 16;   // V^T row pitch (bytes)
  static constexpr int K_BYTES = KT * KP;
  static constexpr int V_BYTES = D * VP + (FP8PV ? 256 : 0);
  static constexpr int BYTES = K_BYTES + V_BYTES;         // one buffer
  static constexpr int K_CHUNKS = D * KE / 16;            // 16-byte chunks per K row
  static constexpr int V_CHUNKS = FP8PV ? KT / 16 : KT / 8;   // 16-byte chunks per V^T row
  static constexpr int K_LOADS = KT * K_CHUNKS;           // 16-byte loads per sub-tile
  static constexpr int V_LOADS = D * V_CHUNKS + (FP8PV ? 16 : 0);
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
template <int D, int CQ, int CK, bool DENSE, bool FP8, int KSPL, bool FP8PV>
__global__ __launch_bounds__(2 * CQ * KSPL) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd(AttnArgs a) {
  using TL = AttnTile<D, FP8, FP8PV>;
  static_assert(!FP8PV || (FP8 && KSPL == 1), "FP8 values need FP8 keys and whole 64-key sub-tiles per wave");
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
  const int bt = attn_kt(a, bh);   // the head whose key tiles and centroids bh reads
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
  constexpr int KLPT = (TL::K_LOADS + NT - 1) / NT, VLPT = (TL::V_LOADS + NT - 1) / NT;
  constexpr bool K_ALL = TL::K_LOADS % NT == 0, V_ALL = TL::V_LOADS % NT == 0;
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
      const int64_t row = ((int64_t)bt * nc + j) * CK + part * TL::KT;
      if constexpr (FP8) {
        ks = reinterpret_cast<const u32x4_t*>(a.kc8 + row * D);
        ksc_nxt = a.kscale[((int64_t)bt * nc + j) * SUB + part];
      } else {
        ks = reinterpret_cast<const u32x4_t*>(a.kc + row * D);
      }
      if constexpr (FP8PV)
        vs = reinterpret_cast<const u32x4_t*>(a.vt8 + (((int64_t)bt * nc + j) * SUB + part) * vt8_bytes<D>());
      else
        vs = reinterpret_cast<const u32x4_t*>(a.vt + (((int64_t)bt * nc + j) * SUB + part) * (int64_t)D * TL::KT);
    } else {
      const int ct = t - Tm;
      if constexpr (FP8) {
        ks = reinterpret_cast<const u32x4_t*>(a.kbar8 + ((int64_t)bt * ncp + ct * TL::KT) * D);
        ksc_nxt = a.kbscale[(int64_t)bt * (ncp / TL::KT) + ct];
      } else {
        ks = reinterpret_cast<const u32x4_t*>(a.kbar_hi + ((int64_t)bt * ncp + ct * TL::KT) * D);
      }
      if constexpr (FP8PV)
        vs = reinterpret_cast<const u32x4_t*>(a.vbar8 + ((int64_t)bt * (ncp / TL::KT) + ct) * vt8_bytes<D>());
      else
        vs = reinterpret_cast<const u32x4_t*>(a.vbar_t + ((int64_t)bt * (ncp / TL::KT) + ct) * D * TL::KT);
    }
#pragma unroll
    for (int i = 0; i < KLPT; ++i)
      if (K_ALL || i * NT + tid < TL::K_LOADS) kst[i] = ks[i * NT + tid];
#pragma unroll
    for (int i = 0; i < VLPT; ++i)
      if (V_ALL || i * NT + tid < TL::V_LOADS) vst[i] = vs[i * NT + tid];
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
      if (V_ALL || e < TL::V_LOADS) {
        // FP8 values: the chunks past the D rows are the scale bytes
        const int off = (FP8PV && e >= D * TL::V_CHUNKS)
                            ? D * TL::VP + (e - D * TL::V_CHUNKS) * 16
                            : (e / TL::V_CHUNKS) * TL::VP + (e % TL::V_CHUNKS) * 16;
        *reinterpret_cast<u32x4_t*>(base + TL::K_BYTES + off) = vst[i];
      }
    }
  };
  // per-lane LDS read bases: K row r, chunk h (FP8: 32-byte chunk h); V^T
  // row r, chunk h
  const int kread = r * TL::KP + h * (FP8 ? 32 : 16);
  const int vread = TL::K_BYTES + r * TL::VP + h * (FP8PV ? 32 : 16);
  const float* logn = a.logn + (int64_t)bt * ncp;

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
      if constexpr (FP8PV) {
        // P as e4m3 codes (P <= 2^8: inside the format's range, no scale).
        // Word q of key block kb holds keys 32 kb + 8 q + 4 h + 0..3 in lane
        // half h; swapping words q = 0, 1 of the upper half with words 2, 3
        // of the lower half gives lane half h keys 32 kb + 16 h + 0..15 of
        // both blocks, in the byte order of the FP8 value rows.
        uint32_t wk[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            wk[kb][q] = e4m3_pack4_raw(tv[16 * kb + 4 * q], tv[16 * kb + 4 * q + 1],
                                       tv[16 * kb + 4 * q + 2], tv[16 * kb + 4 * q + 3]);
        i32x8_t pb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const auto sw = __builtin_amdgcn_permlane32_swap(wk[kb][q], wk[kb][q + 2], false, false);
            pb[4 * kb + 2 * q] = (int)sw[0];
            pb[4 * kb + 2 * q + 1] = (int)sw[1];
          }
        float ps4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 32; ++i) ps4[i & 3] += tv[i];
        lsum += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);   // this lane's keys, fp32 weights
        // O^T block nb += V^T rows 32 nb + r (bytes 32 h .. 32 h + 31) x P^T;
        // this lane half supplies the scales of key block h of rows 32 nb + r
        // (byte nb of one word)
        const int sword = *reinterpret_cast<const int*>(buf + TL::K_BYTES + D * TL::VP + (h * 32 + r) * 4);
        auto vrow = [&](int nb) {
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(buf + vread + nb * 32 * TL::VP);
          const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(buf + vread + nb * 32 * TL::VP + 16);
          return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        acc[0] = mfma32_fp8_scale_a<0>(vrow(0), pb, acc[0], sword);
        acc[1] = mfma32_fp8_scale_a<1>(vrow(1), pb, acc[1], sword);
        if constexpr (NB > 2) {
          acc[2] = mfma32_fp8_scale_a<2>(vrow(2), pb, acc[2], sword);
          acc[3] = mfma32_fp8_scale_a<3>(vrow(3), pb, acc[3], sword);
        }
      } else {
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
      }   // bf16 P.V
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

// ----------------------------------------------------------------------------
// Attention, bf16, software-pipelined (query clusters of 128 or 256)
// ----------------------------------------------------------------------------

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, expanded at compile
// time (a loop the unroller may decline to flatten is not acceptable inside a
// hand-scheduled region)
template <class F, int... I>
CA_DEV void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
CA_DEV void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// 16 bytes per lane from global memory straight into LDS (lane l's bytes land
// at lds + 16 l; lds is wave-uniform). Written out so that the compiler,
// which would otherwise wait for the transfer before every later LDS read,
// leaves the wait to the caller (s_waitcnt vmcnt before the barrier that
// publishes the buffer). M0, which holds the LDS address, is declared
// clobbered: nothing else in the kernels that use this keeps a value in it.
CA_DEV void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}

// Same work as attn_fwd<D, CQ, CK, DENSE, false, 1>, scheduled as a pipeline:
// iteration t computes the softmax of sub-tile t while the matrix cores run
// the Q.K^T products of sub-tile t + 1 and the P.V products of sub-tile
// t - 1. K and V^T sub-tiles are moved into LDS by direct global-to-LDS loads
// (no register staging), double buffered: K of sub-tile t + 2 and V^T of
// sub-tile t are issued at the top of iteration t and waited for at its end,
// one barrier per iteration. LDS rows are unpadded with their 16-byte chunks
// XOR-swizzled by the row index (conflict-free operand reads). The running
// maximum is lazy as in attn_fwd (it moves only when a sub-tile exceeds it by
// more than kLazy); the sub-tile's maximum is taken first, so the weights are
// formed once, against the final value.
//
// LDS of attn_fwd2 past the K and V double buffers: the selected clusters
// (up to kBlkCache entries), then the key bias rows that the Q.K^T
// accumulators start from (in units of the raw score q.k): a zero row for
// whole token sub-tiles, one row per sub-tile of the last, short cluster
// (0, or -inf past its end), and with compensation the centroid bias
// (ln n_c / scale, -inf for selected or padding clusters).
constexpr int kBlkCache = 1024;
struct Attn2Lds {
  int blk_off, bias_off, bytes;
};
template <int D>
Attn2Lds attn2_lds(int nc, int topk, bool comp, int sub) {
  Attn2Lds r;
  r.blk_off = 2 * (64 * 2 * D) + 2 * (D * 2 * 64);
  r.bias_off = (r.blk_off + 4 * std::min(topk, kBlkCache) + 15) / 16 * 16;
  r.bytes = r.bias_off + 4 * 64 * (1 + sub) + (comp ? 4 * attn_ncp(nc) : 0);
  return r;
}

// QS workgroups share a query cluster, each taking CQ / QS of its queries
// (d = 64 with 256-query clusters: two four-wave workgroups instead of one
// of eight, so that three of them fit a CU at three waves per SIMD).
template <int D, int CQ, int CK, bool DENSE, int QS>
__global__ __launch_bounds__(2 * CQ / QS) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2)))
void attn_fwd2(AttnArgs a, Attn2Lds lay) {
  constexpr int NT = 2 * CQ / QS, NW = NT / 64;
  constexpr int KT = 64, KS = D / 16, NB = D / 32, SUB = CK / KT;
  constexpr int KROW = 2 * D, CPRK = KROW / 16;       // K row bytes, 16-byte chunks per row
  constexpr int KBUF = KT * KROW;
  constexpr int VROW = 2 * KT, CPRV = VROW / 16;      // V^T row bytes (64 keys), chunks
  constexpr int VBUF = D * VROW;
  constexpr int KPW = KBUF / 1024 / NW, VPW = VBUF / 1024 / NW;   // 1 KB transfers per wave
  static_assert(KBUF % (1024 * NW) == 0 && VBUF % (1024 * NW) == 0, "whole transfers per wave");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* sBlk = reinterpret_cast<int*>(smem + lay.blk_off);
  float* sKB = reinterpret_cast<float*>(smem + lay.bias_off);   // key bias rows
  float* sBias = sKB + 64 * (1 + SUB);                           // centroid bias
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int G = gridDim.x * gridDim.y;
  const int lg = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, G);
  const int nc = a.nc, nqc = a.nqc, N = a.N;
  const int qa = lg / QS % nqc, bh = lg / QS / nqc, qpart = lg % QS;
  const int bt = attn_kt(a, bh);   // the head whose key tiles and centroids bh reads
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, r = l & 31;
  const int qpos = qa * CQ + qpart * (CQ / QS) + w * 32 + r;
  const bool qvalid = qpos < N;
  const int qtok =
      qvalid ? (DENSE || !a.perm_q ? qpos : clamp_tok(a.perm_q[(int64_t)bh * N + qpos], N)) : 0;
  const uint16_t* Qh = (const uint16_t*)a.Q + (int64_t)bh * N * D;

  bf16x8_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (qvalid) v = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)qtok * D + s * 16 + h * 8);
    qf[s] = as_bf16x8(v);
  }
  floatx16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = zero16();
  float m = kNegInf, lsum = 0.0f;
  const float sl2 = a.scale * kLog2e;

  const int nsel = DENSE ? nc
                  : (a.nsel ? min(max(a.nsel[(int64_t)bh * nqc + qa], 0), a.topk) : a.topk);
  const int32_t* blk = DENSE ? nullptr : a.blocks + ((int64_t)bh * nqc + qa) * a.topk;
  const int Tm = nsel * SUB;
  const int ncp = attn_ncp(nc);
  const bool comp = !DENSE && a.compensate;
  const int T = Tm + (comp ? ncp / KT : 0);
  const int ncache = min(nsel, kBlkCache);
  if (!DENSE) {
    for (int e = tid; e < ncache; e += NT) sBlk[e] = blk[e];
    if (comp) {
      // bias of centroid c: ln n_c / scale if c is not selected, else -inf
      // (the logit scale * (q.kbar_c + bias) is then scale q.kbar_c + ln n_c)
      const float* logn = a.logn + (int64_t)bt * ncp;
      const float inv_scale = 1.0f / a.scale;
      for (int e = tid; e < ncp; e += NT) sBias[e] = logn[e] * inv_scale;
      __syncthreads();
      for (int e = tid; e < nsel; e += NT) {
        const int j = blk[e];
        if (j >= 0 && j < nc) sBias[j] = kNegInf;
      }
    }
  }
  {
    // the zero row, and the rows of the last cluster's sub-tiles: key k of
    // sub-tile u is past the cluster's end when k >= its valid count
    const int last_valid = N - (nc - 1) * CK;   // members of the last cluster
    for (int e = tid; e < 64 * (1 + SUB); e += NT) {
      const int u = e / 64 - 1, k = e % 64;
      sKB[e] = (u < 0 || k < last_valid - u * KT) ? 0.0f : kNegInf;
    }
  }
  __syncthreads();

  // cluster of token sub-tile t, uniform (-1: an out-of-range entry, skipped).
  // The selection is read-only and its address uniform, so the entry comes
  // through the scalar cache into a scalar register: no LDS read, no
  // readfirstlane, and no wait that joins the vector-memory counter.
  const __attribute__((address_space(4))) int32_t* blk4 =
      (const __attribute__((address_space(4))) int32_t*)(uintptr_t)(DENSE ? a.blocks : blk);
  auto valid_cluster = [&](int j) -> int { return (j >= 0 && j < nc) ? j : -1; };
  auto raw_cluster = [&](int t) -> int { return DENSE ? t / SUB : blk4[t / SUB]; };
  auto tile_cluster = [&](int t) -> int { return valid_cluster(raw_cluster(t)); };
  auto uniform_ptr = [](const void* p) -> const unsigned char* {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const unsigned char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
  };
  auto k_src = [&](int t, int j) -> const unsigned char* {
    if (t < Tm)
      return uniform_ptr(a.kc + (((int64_t)bt * nc + max(j, 0)) * CK + (t % SUB) * KT) * D);
    return uniform_ptr(a.kbar_hi + ((int64_t)bt * ncp + (t - Tm) * KT) * D);
  };
  auto v_src = [&](int t, int j) -> const unsigned char* {
    if (t < Tm)
      return uniform_ptr(a.vt + (((int64_t)bt * nc + max(j, 0)) * SUB + t % SUB) * (int64_t)D * KT);
    return uniform_ptr(a.vbar_t + ((int64_t)bt * (ncp / KT) + (t - Tm)) * D * KT);
  };
  // LDS rows keep their 16-byte chunks XOR-swizzled: chunk c of row `row`
  // sits at position c ^ swz(row), swz(row) = (row / RPB) % CPR with RPB the
  // rows per 256 bytes (one pass of the 64 four-byte banks). The 16 lanes that
  // one ds_read_b128 pass serves read rows r .. r + 15 at one chunk, and hit
  // 16 distinct 16-byte bank groups.
  constexpr int RPBK = 256 / KROW > 0 ? 256 / KROW : 1, RPBV = 256 / VROW > 0 ? 256 / VROW : 1;
  auto swz_k = [](int row) { return (row / RPBK) % CPRK; };
  auto swz_v = [](int row) { return (row / RPBV) % CPRV; };
  // per-lane source offsets of this wave's transfers: LDS chunk q = 64 (i NW + w) + l
  // holds row q / CPR, source chunk (q % CPR) ^ swz(row). Transfer i is
  // transfer 0 moved by 1024 NW bytes at both ends: 64 NW chunks are a whole
  // number of rows, and swz does not change over that many rows.
  static_assert((64 * NW / CPRK) % (RPBK * CPRK) == 0 && (64 * NW / CPRV) % (RPBV * CPRV) == 0,
                "transfer stride");
  uint32_t koff, voff;
  {
    const int q = 64 * w + l;
    koff = (q / CPRK) * KROW + ((q % CPRK) ^ swz_k(q / CPRK)) * 16;
    voff = (q / CPRV) * VROW + ((q % CPRV) ^ swz_v(q / CPRV)) * 16;
  }
  // transfer i's per-lane source offsets, loop-invariant: the source base
  // of a sub-tile is then one scalar pair for all of its transfers (no 64-bit
  // scalar add per transfer)
  uint32_t koffs[KPW], voffs[VPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) koffs[i] = koff + 1024 * NW * i;
#pragma unroll
  for (int i = 0; i < VPW; ++i) voffs[i] = voff + 1024 * NW * i;
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds0 + 1024 * w);
  auto load_k = [&](int t, int slot) {
    const unsigned char* src = k_src(t, t < Tm ? tile_cluster(t) : 0);
#pragma unroll
    for (int i = 0; i < KPW; ++i) dma16(koffs[i], src, wlds + slot * KBUF + 1024 * NW * i);
  };
  // per-lane operand read offsets: K row 32 kb + r chunk 2 s + h; V^T row 32 nb + r chunk 2 q + h
  // (LDS addresses: the slot and block offsets of a read are then immediates)
  // K: chunk (2 s + h) ^ x of row r, x = swz_k(r), is at byte
  // 32 (s ^ (x >> 1)) + 16 (h ^ (x & 1)) of the row: kbase + (32 s ^ kx).
  // The per-read XOR (one v_xad with the add) replaces eight address
  // registers that would be loop-invariant and, at this register budget,
  // spilled. (Rows 32 kb + r have the swizzle of row r: 32 is a multiple of
  // RPB * CPR.)
  static_assert(32 % (RPBK * CPRK) == 0 && 32 % (RPBV * CPRV) == 0, "block rows keep the swizzle");
  const uint32_t kbase = lds0 + r * KROW + 16 * (h ^ (swz_k(r) & 1));
  const uint32_t kx = 32 * (swz_k(r) >> 1);
  auto kro_at = [&](uint32_t kxv, int s) -> uint32_t { return kbase + ((32u * s) ^ kxv); };
  uint32_t vro[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) vro[q] = lds0 + 2 * KBUF + r * VROW + (((2 * q + h) ^ swz_v(r)) * 16);
  auto lds16 = [](uint32_t addr) -> bf16x8_t {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>((uintptr_t)addr);
  };

  // accumulator start of sub-tile u's logits: its key bias row (uniform
  // offset in floats into the rows; rpos is set below, before any call)
  int rpos = -1;
  auto kb_row = [&](int u) -> int {
    if (u >= T) return 0;
    if (u >= Tm) return 64 * (1 + SUB) + (u - Tm) * KT;
    if (rpos >= 0 && u / SUB == rpos) return 64 * (1 + u % SUB);
    return 0;
  };
  auto kb_init = [&](int u, floatx16_t (&s2)[2]) __attribute__((always_inline)) {
    const __attribute__((address_space(3))) float* row =
        (const __attribute__((address_space(3))) float*)sKB + kb_row(u);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4_t v = *reinterpret_cast<const __attribute__((address_space(3))) floatx4_t*>(
            row + kb * 32 + 8 * q + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) s2[kb][4 * q + e] = v[e];
      }
  };
  // Q.K^T of sub-tile u in K slot `slot` into s2 (two 32-key blocks)
  auto qk = [&](int u, int slot, floatx16_t (&s2)[2]) __attribute__((always_inline)) {
    kb_init(u, s2);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      const bf16x8_t kv = lds16(kro_at(kx, i >> 1) + slot * KBUF + (i & 1) * 32 * KROW);
      s2[i & 1] = mfma32(kv, qf[i >> 1], s2[i & 1]);
    }
  };
  // the short last cluster's sub-tiles need key masking: rpos is its entry in
  // the selection (every entry of the dense pass)
  if (N % CK != 0) {
    if (DENSE) {
      rpos = nc - 1;
    } else {
      int mine = -1;
      for (int e = l; e < nsel; e += 64)
        if ((e < kBlkCache ? sBlk[e] : blk[e]) == nc - 1) mine = e;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mine = max(mine, __shfl_xor(mine, o, 64));
      rpos = __builtin_amdgcn_readfirstlane(mine);
    }
  }
  // Logits (two 32-key blocks) and bf16 weights of sub-tile t live in
  // S[t & 1] and PK[t & 1]: with the parity of t known at compile time, each
  // iteration reads one set and writes the other (no copies), and every LDS
  // slot offset is an immediate.
  floatx16_t S[2][2];
  bf16x8_t PK[2][4];
  // clusters of sub-tiles t, t + 1 and t + 2 (uniform; 0 for centroid
  // sub-tiles and past the end), read one iteration ahead as they are stored
  // in the selection and checked where they are used (-1 for an entry out of
  // range: a skipped sub-tile), so that the scalar load of an iteration's
  // last entry completes during its transfer wait and barrier
  auto cl = [&](int t) -> int { return t < Tm ? raw_cluster(t) : 0; };
  int jc0 = cl(0), jc1 = cl(1), jc2 = cl(2);
  const int jc_last = T > 0 ? valid_cluster(cl(T - 1)) : 0;
  // prologue: K of sub-tiles 0 and 1, Q.K^T of sub-tile 0; zero weights and
  // a zeroed V^T slot 1 for the P.V products of iteration 0
  if (T > 0) {
    load_k(0, 0);
    load_k(T > 1 ? 1 : 0, 1);   // finite data in slot 1 even for a single sub-tile
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) PK[1][q] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
  for (int e = tid; e < VBUF / 16; e += NT)
    *reinterpret_cast<u32x4_t*>(smem + 2 * KBUF + VBUF + 16 * e) = u32x4_t{0u, 0u, 0u, 0u};
  __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
  __syncthreads();
  if (T > 0) qk(0, 0, S[0]);
  __syncthreads();   // every wave has read K slot 0 before it is refilled

  // Iteration t (parity P = t & 1): one straight-line region holding the
  // transfers for later sub-tiles, the P.V products of t - 1 (PV), the Q.K^T
  // products of t + 1 (QK) and the softmax of t, then the rare rescale, the
  // wait for the transfers and the barrier.
  auto iter = [&](int t, auto parity, auto pv_tag, auto qk_tag) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value;
    floatx16_t (&scur)[2] = S[P];
    floatx16_t (&snext)[2] = S[P ^ 1];
    const bf16x8_t (&pkold)[4] = PK[P ^ 1];
    bf16x8_t (&pk)[4] = PK[P];
    const int j0 = valid_cluster(jc0);
    const bool skip = t >= T || j0 < 0;
    // transfers of this iteration (issued inside the region below): V^T of
    // sub-tile t into V slot P and K of sub-tile t + 2 into K slot P. Past
    // the last sub-tile both repeat the last V^T tile's 16 KB source (the
    // slots are read again only by products whose results are discarded or
    // multiplied by zero weights), which keeps the region free of branches.
    const unsigned char* vsrc = t < T ? v_src(t, j0) : v_src(T - 1, max(jc_last, 0));
    const unsigned char* ksrc = t + 2 < T ? k_src(t + 2, valid_cluster(jc2)) : vsrc;
    const float skipoff = skip ? kNegInf : 0.0f;   // uniform: no branch in the region
    const float scl = sl2;
    // One instruction stream in a fixed order (scheduling barriers between
    // steps): step i issues product i (the 4 NB P.V products of t - 1, then
    // the 2 KS Q.K^T products of t + 1) and the LDS read of product i + PF's
    // operand, beside the softmax of sub-tile t: its maximum over the first
    // MS steps, then (branch-free, per lane) the new running maximum, and in
    // the remaining steps the weights against it, packed to bf16 and summed
    // 8 at a time. Nothing of sub-tile t's logits is needed afterwards.
    constexpr int NPV = PV ? 4 * NB : 0, NM = NPV + (QK ? 2 * KS : 0);
    constexpr int PF = 4;
    constexpr int NSTEP = NM > 0 ? NM : 1;
    constexpr int MS = NSTEP >= 4 ? NSTEP / 4 : 1;        // steps of the maximum
    constexpr int E0 = NSTEP > 1 ? MS : 0, NE = NSTEP - E0;   // steps of the weights
    uint32_t kxo = kx;
    asm volatile("" : "+v"(kxo));   // opaque: the K read addresses stay in the loop
    auto operand = [&](int i) -> bf16x8_t {
      if (i < NPV) {
        const int nb = i % NB, q = i / NB;
        return lds16(vro[q] + (P ^ 1) * VBUF + nb * 32 * VROW);
      }
      const int k = i - NPV;
      return lds16(kro_at(kxo, k >> 1) + (P ^ 1) * KBUF + (k & 1) * 32 * KROW);
    };
    bf16x8_t ring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (i < NM) ring[i] = operand(i);
    // the products of t + 1 accumulate onto the bias row; its reads go after
    // the first operands (LDS reads return in order, and the Q.K^T products
    // come after the P.V ones), so the first product waits for its operand only
    if constexpr (QK) kb_init(t + 1, snext);
    float ps = 0.0f, tv[8], bm = kNegInf, mn = m, nm = 0.0f;
    static_for<NSTEP>([&](auto step) __attribute__((always_inline)) {
      constexpr int i = decltype(step)::value;
      __builtin_amdgcn_sched_barrier(0);
      // one transfer per step from the first (V^T first: it is needed sooner)
      static_for<VPW + KPW>([&](auto xc) __attribute__((always_inline)) {
        constexpr int x = decltype(xc)::value;
        if constexpr ((x < NSTEP ? x : NSTEP - 1) == i) {
          if constexpr (x < VPW) dma16(voffs[x], vsrc, wlds + 2 * KBUF + P * VBUF + 1024 * NW * x);
          else dma16(koffs[x - VPW], ksrc, wlds + P * KBUF + 1024 * NW * (x - VPW));
        }
      });
      if constexpr (i < NPV) {
        acc[i % NB] = mfma32(ring[i % PF], pkold[i / NB], acc[i % NB]);
      } else if constexpr (i < NM) {
        constexpr int k = i - NPV;
        snext[k & 1] = mfma32(ring[i % PF], qf[k >> 1], snext[k & 1]);
      }
      if constexpr (i + PF < NM) ring[i % PF] = operand(i + PF);
      static_for<32>([&](auto ec) __attribute__((always_inline)) {
        constexpr int el = decltype(ec)::value;
        if constexpr (el * MS / 32 == i) bm = fmaxf(bm, scur[el >> 4][el & 15]);
      });
      if constexpr (i == MS - 1) {
        // the lazy maximum: it moves only when the sub-tile exceeds it by
        // more than kLazy (always for the first sub-tile with keys); a
        // skipped sub-tile gets weight 0 through the offset -inf
        bm = max_halves(bm) * scl;
        mn = ((bm > m + kLazy) & !skip) ? bm : m;
        nm = (mn == kNegInf ? 0.0f : -mn) + skipoff;
      }
      static_for<32>([&](auto ec) __attribute__((always_inline)) {
        constexpr int el = decltype(ec)::value;
        if constexpr (i >= E0 && E0 + el * NE / 32 == i) {
          tv[el & 7] = __builtin_amdgcn_exp2f(fmaf(scur[el >> 4][el & 15], scl, nm));
          if constexpr ((el & 7) == 7) {
            u32x4_t u = pack8(tv);
            ps = sum_bf16x8(u, ps);
            // pinned here: left free, the weights sink past the rescale
            // branch, out of the interleaved region
            asm volatile("" : "+v"(u), "+v"(ps));
            pk[el >> 3] = as_bf16x8(u);
          }
        }
      });
    });
    __builtin_amdgcn_sched_barrier(0);
    if (__ballot(mn != m)) [[unlikely]] {
      // the maximum moved: rescale what is accumulated (the P.V products of
      // t - 1 are in)
      const float alpha = mn != m ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][i] *= alpha;
      m = mn;
    }
    lsum += ps;
    jc0 = jc1;
    jc1 = jc2;
    jc2 = cl(t + 3);
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this iteration's transfers
    __syncthreads();
  };
  // Iterations t = 0 .. T: every one runs the whole pipeline. Iteration 0's
  // P.V products multiply zero weights with a zeroed V^T slot; sub-tiles from
  // T on are skipped (weight 0) and their Q.K^T products discarded, so
  // iteration T only completes the P.V products of T - 1 (and one more
  // padding iteration follows when T is odd). With no remainder variants of
  // the iteration every value stays in registers.
  using T_ = std::true_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (T > 0) {
    iter(0, P0{}, T_{}, T_{});
#pragma unroll 1
    for (int t = 1; t <= T; t += 2) {
      iter(t, P1{}, T_{}, T_{});
      iter(t + 1, P0{}, T_{}, T_{});
    }
  }

  lsum = sum_halves(lsum);
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


template <int D, bool FP8, bool FP8PV>
constexpr size_t attn_smem() {
  return 2 * (size_t)AttnTile<D, FP8, FP8PV>::BYTES + 8192 / 8 + 64;   // two buffers, selection bits
}

// ----------------------------------------------------------------------------
// fp32 path
// ----------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void centroids_kv_f32(AttnArgs a) {
  const int j = blockIdx.x, bh = blockIdx.y * (a.kshare > 1 ? a.kshare : 1);   // heads that build tiles
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
  const int bt = attn_kt(a, bh);   // the head whose key clusters and centroids bh reads
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
          const int tok = DENSE ? pos : clamp_tok(a.perm_k[(int64_t)bt * N + pos], N);
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
      const float* kb = a.kbar32 + ((int64_t)bt * ncp + j) * D;
      const float* vb = a.vbar32 + ((int64_t)bt * ncp + j) * D;
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s += q[d] * kb[d];
      absorb(s * a.scale + a.logn[(int64_t)bt * ncp + j], vb);
    }
  }
  if (!qvalid) return;
  float* Oh = (float*)a.O + ((int64_t)bh * N + qtok) * D;
  const float inv = 1.0f / lsum;
  for (int d = 0; d < D; ++d) Oh[d] = o[d] * inv;
  if (a.lse) a.lse[(int64_t)bh * N + qtok] = m + logf(lsum);
}

template <int D, int CQ, int CK, bool DENSE, bool FP8, bool FP8PV>
void launch_mfma(const AttnArgs& a, hipStream_t st) {
  constexpr int KSPL = CQ == 64 ? 2 : 1;
  const size_t sm = attn_smem<D, FP8, FP8PV>();
  CA_MAX_LDS_ONCE((&attn_fwd<D, CQ, CK, DENSE, FP8, KSPL, FP8PV>), sm);
  dim3 g(a.nqc, a.BH);
  if (a.ev_start) (void)hipEventRecord(a.ev_start, st);
  attn_fwd<D, CQ, CK, DENSE, FP8, KSPL, FP8PV><<<g, 2 * CQ * KSPL, sm, st>>>(a);
  if (a.ev_stop) (void)hipEventRecord(a.ev_stop, st);
}

// bf16 without FP8 operands, query clusters of 128 or 256: the pipelined kernel
template <int D, int CQ, int CK, bool DENSE>
void launch_mfma2(const AttnArgs& a, hipStream_t st) {
  constexpr int QS = (D == 64 && CQ == 256) ? 2 : 1;
  const Attn2Lds lay = attn2_lds<D>(a.nc, DENSE ? 0 : a.topk, !DENSE && a.compensate, CK / 64);
  CA_MAX_LDS_ONCE((&attn_fwd2<D, CQ, CK, DENSE, QS>), 160 * 1024);
  dim3 g(a.nqc * QS, a.BH);
  if (a.ev_start) (void)hipEventRecord(a.ev_start, st);
  attn_fwd2<D, CQ, CK, DENSE, QS><<<g, 2 * CQ / QS, (size_t)lay.bytes, st>>>(a, lay);
  if (a.ev_stop) (void)hipEventRecord(a.ev_stop, st);
}

template <int D, bool FP8, bool FP8PV>
void launch_tiles(const AttnArgs& a, bool dense, hipStream_t st) {
  // tiles of the heads that build them (every head, or each key-sharing
  // group's first head)
  const int tile_heads = a.BH / (a.kshare > 1 ? a.kshare : 1);
  dim3 gp(attn_ncp(a.nc), tile_heads);
  permute_kv<D, FP8, FP8PV><<<gp, 256, 0, st>>>(a);
  if (FP8 && !dense && a.compensate) {
    dim3 gq(attn_ncp(a.nc) / 64, tile_heads);
    quant_centroids<D><<<gq, 256, 0, st>>>(a);
    if (FP8PV) quant_vcentroids<D><<<gq, 256, 0, st>>>(a);
  }
  if (dense) {
    if constexpr (!FP8) launch_mfma2<D, 128, 128, true>(a, st);
    else launch_mfma<D, 128, 128, true, FP8, FP8PV>(a, st);
    return;
  }
  // (query, key) cluster sizes: equal, or the key clusters larger (FP8
  // values: query clusters of at least 128, checked on the host)
  if constexpr (FP8PV) {
    switch (a.cq * 1000 + a.c) {
      case 128128: launch_mfma<D, 128, 128, false, FP8, FP8PV>(a, st); break;
      case 128256: launch_mfma<D, 128, 256, false, FP8, FP8PV>(a, st); break;
      default: launch_mfma<D, 256, 256, false, FP8, FP8PV>(a, st); break;
    }
  } else if constexpr (!FP8) {
    switch (a.cq * 1000 + a.c) {
      case 64064: launch_mfma<D, 64, 64, false, FP8, FP8PV>(a, st); break;
      case 64128: launch_mfma<D, 64, 128, false, FP8, FP8PV>(a, st); break;
      case 64256: launch_mfma<D, 64, 256, false, FP8, FP8PV>(a, st); break;
      case 128128: launch_mfma2<D, 128, 128, false>(a, st); break;
      case 128256: launch_mfma2<D, 128, 256, false>(a, st); break;
      default: launch_mfma2<D, 256, 256, false>(a, st); break;
    }
  } else {
    switch (a.cq * 1000 + a.c) {
      case 64064: launch_mfma<D, 64, 64, false, FP8, FP8PV>(a, st); break;
      case 64128: launch_mfma<D, 64, 128, false, FP8, FP8PV>(a, st); break;
      case 64256: launch_mfma<D, 64, 256, false, FP8, FP8PV>(a, st); break;
      case 128128: launch_mfma<D, 128, 128, false, FP8, FP8PV>(a, st); break;
      case 128256: launch_mfma<D, 128, 256, false, FP8, FP8PV>(a, st); break;
      default: launch_mfma<D, 256, 256, false, FP8, FP8PV>(a, st); break;
    }
  }
}

template <int D>
void launch_bf16(const AttnArgs& a, bool dense, hipStream_t st) {
  if (a.dtype == 3) launch_tiles<D, true, true>(a, dense, st);
  else if (a.dtype == 2) launch_tiles<D, true, false>(a, dense, st);
  else launch_tiles<D, false, false>(a, dense, st);
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
  dim3 gc(attn_ncp(a.nc), a.BH / (a.kshare > 1 ? a.kshare : 1));   // the centroid-building heads
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
