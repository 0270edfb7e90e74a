// Launch wrappers of the gfx950 kernels (host side, called by ca_api.hip).
#pragma once

#include "common.h"

namespace ca {

// metric.hip -----------------------------------------------------------------
int metric_rows_per_chunk(int N, int BH);
// dtype: 0 = bf16, 1 = fp32. partial: [BH][nchunks][2 D D + D] fp32 scratch.
// M_q, M_k, kbar, the query geometry's bf16 split and the row hashes
void launch_metric(const void* Q, const void* K, int dtype, int BH, int N, int D, int transform,
                   float* partial, uint64_t* hash, float* Mq, float* Mk, float* kbar,
                   uint16_t* gsplit, float* Mpk, int kvg, hipStream_t st);
// the query normalisers s [BH][N] (1 without query normalisation), after launch_metric
void launch_qnorm(const void* Q, int dtype, int BH, int N, int D, int transform,
                  int query_normalize, const uint16_t* gsplit, const float* Mk, float* s,
                  hipStream_t st);
// kvg: query heads per key/value head (1 = multi-head attention); the key
// rows of query head bh are those of key/value head bh / kvg (every call).

// cluster.hip ----------------------------------------------------------------
struct LevelArgs {
  const void* Q;
  const void* K;
  int dtype;
  int BH, N, D, c, level;
  int kvg;                  // query heads per key/value head (key rows of tree 2 bh + 1: head bh / kvg)
  int transform, power_iters, sample_factor;
  int split_mode;           // 0 = power iteration, 1 = diagonalized (basis below)
  int tree_step, tree_base; // trees of this launch: blockIdx.y * tree_step + tree_base
                            // (1, 0: all 2 BH; 2, t: tensor t's BH trees)
  uint64_t seed;
  const int32_t* perm_in;   // [2 BH][N]
  int32_t* perm_out;        // [2 BH][N]
  const uint64_t* hpos_in;  // [2 BH][N] content hash of the token at each position
  uint64_t* hpos_out;       // [2 BH][N] the same after this level's partition
  const float* s;           // [BH][N]
  const float* Mq;          // [BH][D][D]
  const float* Mk;          // [BH][D][D]
  const float* Mpk;         // [2 BH][D D]: metric of each tree (M_k for queries, M_q for
                            // keys) packed in the per-lane order of the direction kernel
  const float* basis;       // [2 BH][D][D]: row j = basis direction a_j (diagonalized)
  const float* Y;           // [2 BH][N][D]: coordinates x . a_j of every token (diagonalized)
  int32_t* jsel;            // [2 BH][node_slots]: chosen coordinate of each node (diagonalized)
  const float* dir_prev;    // [2 BH][node_slots][D], slots of the previous level
  float* dir_cur;           // [2 BH][node_slots][D]
  int node_slots;           // per-tree row stride of jsel and the direction arrays: the
                            // deepest level's slot count, the same at every level so that
                            // trees at different levels (two streams) never share a row
  int nchunks;              // ceil(N / c)
  int sample_inline;        // set by launch_level: the direction kernel draws the subsample itself
  int split_cache;          // set by launch_level: keys a split workgroup keeps in LDS
  int32_t* wide;            // wide split of the large-node levels: per-node state, per-chunk counts
  int wide_cpn;             // set by launch_level: chunks per node of a wide level
  int32_t* sample_buf;      // [2 BH][N]   per-chunk sample lists
  int32_t* chunk_cnt;       // [2 BH][nchunks]
  int32_t* zbuf_tok;        // [2 BH][N]   a node's gathered sample tokens
  float* zbuf;              // [2 BH][N]
  uint32_t* keys;           // [2 BH][N]
  float* trace_score;       // [2 BH][N] or null
  float* trace_dir;         // [2 BH][trace_slots][D] or null
  int trace_slots;
};
void launch_level(const LevelArgs& a, hipStream_t st);
// workspace words (int32) of the wide split of the large-node levels (0: none)
size_t wide_split_words(int BH, int N, int c);

// basis.hip ------------------------------------------------------------------
// Principal-component basis of each tree for diagonalized splitting: At
// [2 BH][D][D] (row j = a_j); partial as for launch_metric, Cq [BH][D][D],
// Rbuf and Zbuf [2 BH][D][D] scratch.
void launch_basis(const void* Q, int dtype, int BH, int N, int D, int transform, const float* s,
                  const float* Mq, const float* Mk, float* partial, float* Cq, float* Rbuf,
                  float* Zbuf, float* At, hipStream_t st);
// Y [2 BH][N][D] = coordinates of every query (s q) and key in its tree's
// basis At; At3 [2 BH][3][D][D] bf16 scratch (bf16 inputs).
void launch_rotate(const void* Q, const void* K, int dtype, int BH, int N, int D, const float* s,
                   const float* At, uint16_t* At3, float* Y, int kvg, hipStream_t st);
void launch_perm_init(int32_t* perm, int trees, int N, hipStream_t st);
// perm [2 BH][N] tree order -> perm_q, perm_k [BH][N]; the query trees are
// read from perm_qt, the key trees from perm_kt
// (kshare > 1: the key trees of heads bh - bh % kshare serve their whole group)
// (tensor 0: perm_q from the query trees, 1: perm_k from the key trees)
void launch_perm_out(const int32_t* perm_t, int tensor, int BH, int N, int kshare, int32_t* perm,
                     hipStream_t st);
// Shared key clustering of groups of g query heads: the key-tree metric of
// the group's first head (Mq and its packed copy in Mpk) becomes the mean of
// the group's query metrics.
void launch_pool_key_metric(float* Mq, float* Mpk, int BH, int D, int g, hipStream_t st);
// centroids of query clusters of size c_q and key clusters of size c_k;
// counts (optional) = key cluster sizes; tensors t0 .. t0 + nt - 1 (0 = queries, 1 = keys)
void launch_centroids(const void* Q, const void* K, int dtype, int BH, int N, int D, int c_q,
                      int c_k, const int32_t* perm_q, const int32_t* perm_k, float* cent_q,
                      float* cent_k, int32_t* counts, int kvg, int t0, int nt, hipStream_t st);

// route.hip ------------------------------------------------------------------
void launch_route(const float* cq, const float* ck, int BH, int nq, int nk, int D, int topk,
                  float* scores, int32_t* blocks, hipStream_t st);
// Scratch of the allocation-free routing call: at most kRouteScratchFloats
// scores (B H n_qc n_kc), 32 MiB per device. route_scratch gives the device
// address of that array on the current device (looked up once per device,
// thread-safe); nonzero with *err set if the lookup fails.
constexpr size_t kRouteScratchFloats = (size_t)8 << 20;
int route_scratch(float** out, const char** err);
// adaptive selection: blocks [BH][nq][nk] (the first nsel entries of a row
// are the selected clusters, ascending; the rest -1), nsel [BH][nq]
void launch_route_adaptive(const float* cq, const float* ck, const int32_t* counts, int BH, int nq,
                           int nk, int D, float tau, double recall, int min_count, float* scores,
                           int32_t* blocks, int32_t* nsel, hipStream_t st);

// attn.hip -------------------------------------------------------------------
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  int dtype;   // 0 bf16, 1 fp32, 2 bf16 with FP8 (e4m3) Q.K^T operands, 3 FP8 Q.K^T and P.V
  int BH, N, D, c, nc, topk, compensate;   // c, nc: key cluster size and count
  int kvg;                                 // query heads per key/value head (K, V rows of head bh / kvg)
  int kshare;                              // query heads sharing one key clustering: the key
                                           // tiles and centroids of head bh are those built
                                           // for head kt(bh) = (bh / kshare) * kshare (1: own)
  int cq, nqc;                             // query cluster size and count
  float scale;
  const int32_t* perm_q;
  const int32_t* perm_k;
  const int32_t* blocks;
  const int32_t* nsel;   // [BH][nc] selected clusters per row of blocks, or null (= topk)
  void* O;
  float* lse;
  // scratch (bf16 path)
  uint16_t* kc;       // [BH][nc][c][D]   keys, cluster-major, zero padded
  uint16_t* vt;       // [BH][nc][D][c]   values, cluster-major, transposed
  uint16_t* kbar_hi;  // [BH][ncp][D]   key centroids rounded to bf16
  uint16_t* vbar_t;   // [BH][ncp/64][D][64] value centroids, transposed per 64
  float* logn;        // [BH][ncp]
  float* kbar32;      // [BH][ncp][D]
  float* vbar32;      // [BH][ncp][D]
  // scratch of the FP8 variant (carved from kc, kbar32 and vbar32)
  uint8_t* kc8;       // [BH][nc][c][D]   key codes, cluster-major, zero padded
  float* kscale;      // [BH][nc][c/64]   one scale per 64-key sub-tile
  uint8_t* kbar8;     // [BH][ncp][D]     key-centroid codes
  float* kbscale;     // [BH][ncp/64]     one scale per 64 centroids
  // FP8 values (dtype 3; carved from vt and from vbar32 past kbscale): per
  // 64-key sub-tile D rows of 64 codes and 256 scale bytes
  uint8_t* vt8;       // [BH][nc][c/64] sub-tiles
  uint8_t* vbar8;     // [BH][ncp/64]   sub-tiles of the value centroids
  // optional events recorded around the main attention kernel
  hipEvent_t ev_start;
  hipEvent_t ev_stop;
};
// centroid count padded to whole 64-centroid sub-tiles
CA_HD int attn_ncp(int nc) { return (nc + 63) / 64 * 64; }
// head whose key tiles and centroids head bh reads
CA_HD int attn_kt(const AttnArgs& a, int bh) { return a.kshare > 1 ? bh / a.kshare * a.kshare : bh; }
void launch_attend(const AttnArgs& a, hipStream_t st);

// peak.hip -------------------------------------------------------------------
void launch_peak_mfma(int blocks, int iters, float* out, hipStream_t st);
void launch_peak_lds(int blocks, int iters, float* out, hipStream_t st);
void launch_dense(const AttnArgs& a, hipStream_t st);
// quant.hip ------------------------------------------------------------------
void launch_quantize_e4m3(const void* X, int dtype, int64_t rows, int D, int group, uint8_t* codes,
                          float* scales, hipStream_t st);

}  // namespace ca
