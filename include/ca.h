/*
 * ca.h -- C ABI of the ClusterAttention forward path for AMD Instinct MI355X
 * (gfx950).
 *
 * The method is the one of "ClusterAttention: A training-free speedup of
 * bidirectional attention" (arXiv 2608.26965): per head, queries and keys are
 * clustered separately by recursive principal-direction splitting into
 * clusters of a fixed size c (v1 §3.1, §3.2); every query cluster selects the
 * top-k key clusters by centroid score (§3.3); queries attend with token
 * resolution to the selected clusters and, optionally, to every excluded
 * cluster through its key and value centroids with weight |c|
 * ("striped mean-compensation", §1.2 Eq. 5-6, App. A Eq. 21-22).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are contiguous, row-major [B, H, N, D] (batch, head, token, dim),
 *    element type given by ca_dtype. D must be 64 or 128.
 *  - Every pointer argument is a device pointer owned by the caller unless it
 *    is documented as a host pointer. The library never allocates device or
 *    host memory, never frees caller memory and keeps no state between calls
 *    except a thread-local error string, with four stated exceptions: the
 *    per-thread profiling events of ca_profile_events (a timing hook outside
 *    the computation, off unless set), the scratch array of ca_route_noalloc
 *    (one per GPU, for callers that cannot allocate), a once-per-process,
 *    thread-safe raise of some kernels' dynamic LDS limit at their first
 *    launch, and the side stream of ca_cluster (one per GPU, with one pair of
 *    fork/join events per host thread and GPU, created at first use).
 *  - Scratch memory is passed in as `ws` (device, 256-byte aligned) of
 *    `ws_bytes` bytes; ca_workspace_size() gives the bytes a call needs.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream): they enqueue kernels and return. The caller synchronises before
 *    reading outputs. No call performs a device-to-host copy or a host sync,
 *    so the sequence can be captured in a HIP graph.
 *  - Inputs are never written. Outputs are completely overwritten.
 *  - Arguments are validated on the host before anything is enqueued: a
 *    non-CA_OK return means nothing was launched and no output was touched.
 *    Errors are reported by return code (no exceptions, no abort); a detail
 *    string is available from ca_last_error().
 *  - Results are deterministic: the same inputs give bitwise identical outputs
 *    (no floating-point atomics; all reductions run in a fixed order).
 */
#ifndef CLUSTERATTN_CA_H
#define CLUSTERATTN_CA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CA_OK = 0,
  CA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, k out of range, ...   */
  CA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (D, c, dtype combo) */
  CA_ERR_WORKSPACE = 3,    /* ws is NULL, misaligned or smaller than needed */
  CA_ERR_HIP = 4           /* a HIP runtime call failed (see ca_last_error) */
} ca_status;

typedef enum {
  CA_BF16 = 0,             /* bfloat16 inputs and outputs, fp32 accumulation */
  CA_F32 = 1,              /* float32 throughout                             */
  CA_BF16_FP8 = 2,         /* attention only (ca_attend*, ca_dense): bfloat16
                              inputs and outputs, the Q.K^T product on FP8
                              (OCP E4M3) operands, P.V as with CA_BF16       */
  CA_BF16_FP8_PV = 3       /* attention only: as CA_BF16_FP8, and P.V on FP8
                              operands too (query clusters of 128 or 256)    */
} ca_dtype;

typedef enum {
  CA_OP_CLUSTER = 0,
  CA_OP_ROUTE = 1,
  CA_OP_ATTEND = 2,
  CA_OP_DENSE = 3,
  CA_OP_CLUSTER_DIAG = 4   /* ca_cluster with split_mode 1 (diagonalized)    */
} ca_op;

/*
 * Options of the clustering (v1 §3.2). Pass NULL for the defaults
 * {transform=1, query_normalize=1, power_iters=8, sample_factor=1, seed=0,
 *  trace_perm=NULL, trace_score=NULL, trace_dir=NULL, split_mode=0,
 *  trace_basis=NULL, cluster_size_k=0, kv_heads=0, kv_share=0}.
 *
 *  transform        1: keys are split under the query metric M_q = Q^T Q / N
 *                   (Eq. 12-14) and queries under the centred key metric
 *                   M_k = K_c^T K_c / N (Eq. 15); the metric is injected into
 *                   the power iteration, so no root matrix is formed.
 *                   0: Euclidean geometry for both.
 *  query_normalize  1: queries are split as s_i q_i, s_i = (q_i^T G q_i)^-1/2
 *                   with G the query geometry (the top-k representation of
 *                   Eq. 16); a query with q^T G q <= 0 gets s_i = 0.
 *  power_iters      p >= 1, power iterations per split (v1 §3.2.1).
 *  sample_factor    a >= 1: each node estimates its direction from a
 *                   Bernoulli sample of expected size min(a D, n) chosen by a
 *                   64-bit hash of each token's raw input row.
 *  seed             salt of the sample and of the warm-start vectors.
 *  trace_perm       optional device buffer int32 [L+1][B*H][2][N]: the
 *                   permutation before each of the L split levels and the
 *                   final one (tensor index 0 = queries, 1 = keys). L is
 *                   ca_tree_levels(N, c).
 *  trace_score      optional device buffer float [L][B*H][2][N]: the
 *                   projection of the token at each position at each level;
 *                   positions inside leaves are left untouched.
 *  trace_dir        optional device buffer float [L][B*H][2][S][D] with
 *                   S = 2^(L-1): the unit direction of the node in slot j of
 *                   level l (slot j's children are slots 2j and 2j+1 of level
 *                   l+1); slots without a splitting node are left untouched.
 *  split_mode       0: basic recursive splitting, each node's direction by
 *                   power iteration (v1 §3.2.1 "Basic recursive splitting").
 *                   1: diagonalized recursive splitting (v1 §3.2.1
 *                   "Diagonalized recursive splitting"; later revision
 *                   §4.1.1): each tree first computes the principal-component
 *                   basis A = R W of its whole set in the tree's geometry (R
 *                   the symmetric root of the geometry with negative
 *                   eigenvalues clamped, W the eigenvectors of R C R with C
 *                   the centred covariance of the split vectors, by
 *                   descending eigenvalue, each signed so that its largest-
 *                   magnitude entry is positive); each node then splits along
 *                   the basis coordinate y_j = x . a_j of highest population
 *                   variance over its sample (lowest j on ties). power_iters
 *                   is ignored. trace_dir then holds the chosen a_j.
 *  trace_basis      optional device buffer float [B*H][2][D][D] (split_mode
 *                   1 only): row j of tree (head, tensor) is a_j.
 *  cluster_size_k   0: keys are clustered with cluster_size like the
 *                   queries; else the key cluster size c_k in {64, 128, 256}
 *                   (the pages pair c_q = 64 with c_k = 128, v1 §3.1). Each
 *                   tensor's tree then follows its own size; the trace
 *                   buffers need equal sizes (else CA_ERR_UNSUPPORTED).
 *  kv_heads         0: K has H heads (multi-head attention). Else K is
 *                   [B, kv_heads, N, D] with kv_heads dividing H (grouped- or
 *                   multi-query attention): query head h shares the key rows
 *                   of head h / (H / kv_heads), and every query head still
 *                   clusters those keys under its own metric, so perm_k,
 *                   cent_k and counts stay per query head (the pages' option
 *                   of one key clustering per associated query head, v1 §6.2
 *                   "Extension beyond MHA"). CA_ERR_INVALID_ARG if kv_heads
 *                   does not divide H.
 *  kv_share         0: as above. 1 (with kv_heads): the pages' other option,
 *                   one key clustering per key/value head under the mean of
 *                   its query heads' metrics M_q; it takes the random draws
 *                   of the group's first query head, and its permutation,
 *                   centroids and counts are written to every query head of
 *                   the group (identical rows), so routing and attention are
 *                   called as before (ca_attend_ex with kv_shared = 1 then
 *                   builds the key tiles once per group).
 */
typedef struct {
  int transform;
  int query_normalize;
  int power_iters;
  int sample_factor;
  uint64_t seed;
  int32_t* trace_perm;
  float* trace_score;
  float* trace_dir;
  int split_mode;
  float* trace_basis;
  int cluster_size_k;
  int kv_heads;
  int kv_share;
} ca_cluster_opts;

/* Number of split levels of the data-independent tree for (N, c): the tree
 * splits a node of n > c members at the multiple of c closest to n/2 (ties to
 * the smaller), v1 §3.2.1. Returns -1 for invalid arguments. Host only. */
int ca_tree_levels(int N, int cluster_size);

/* Bytes of workspace `op` needs for the given sizes (0 if none, SIZE_MAX if
 * the arguments are invalid). For CA_OP_ROUTE pass N = n_qc and
 * cluster_size = n_kc (the bytes are only needed when `scores` is NULL);
 * CA_OP_DENSE ignores cluster_size and topk. CA_OP_CLUSTER_DIAG is the
 * workspace of ca_cluster with split_mode 1: it adds the coordinates of every
 * query and key in its tree's basis (2 B H N D floats). Host only. */
size_t ca_workspace_size(ca_op op, int B, int H, int N, int D, int cluster_size, int topk);

/*
 * ca_cluster -- recursive PDDP clustering of queries and keys (v1 §3.2.1
 * "Basic recursive splitting" with the transforms of §3.2.2; the later
 * revision's §4.1.1 gives the radix split).
 *
 * Q, K      [B,H,N,D] of type dt (device, read only).
 * cluster_size  c in {64, 128, 256}; N >= c; B*H*N < 2^31.
 * perm_q, perm_k  out int32 [B,H,N]: perm[p] = index of the token at
 *           cluster-major position p. Cluster j occupies positions
 *           [j c, j c + n_j); every n_j = c except the last, which holds
 *           N - (n_c - 1) c (v1 §3.1). Members of a cluster are in ascending
 *           token order.
 * cent_q, cent_k  out float [B,H,n_qc,D] and [B,H,n_kc,D], n_qc = ceil(N/c_q),
 *           n_kc = ceil(N/c_k) (c_q = cluster_size, c_k = opts->cluster_size_k
 *           or c_q; below n_c is either): means of the
 *           original (untransformed) query / key rows of each cluster.
 * counts    out int32 [B,H,n_kc] or NULL: n_j of the key clusters.
 * ws        workspace of ca_workspace_size(CA_OP_CLUSTER (CA_OP_CLUSTER_DIAG
 *           for split_mode 1), B, H, N, D, min(c_q, c_k), 0).
 * stream    the query trees' split levels run on `stream`; the key trees'
 *           run beside them on a library-owned side stream of the current
 *           GPU (non-blocking, default priority), which waits for `stream`
 *           at the call's start (an event) and which `stream` waits for
 *           before the centroids (another event). The call is therefore
 *           ordered on `stream` as a whole, and a HIP graph captured on
 *           `stream` holds both branches. Calls from several host threads
 *           share the side stream (correct, but they serialise there); a
 *           capture on one thread must not overlap a ca_cluster call of
 *           another thread on the same GPU.
 */
int ca_cluster(const void* Q, const void* K, ca_dtype dt, int B, int H, int N, int D,
               int cluster_size, const ca_cluster_opts* opts, int32_t* perm_q,
               int32_t* perm_k, float* cent_q, float* cent_k, int32_t* counts, void* ws,
               size_t ws_bytes, void* stream);

/*
 * ca_route -- centroid scoring and top-k selection (v1 §3.3, Eq. 18).
 *
 * cent_q    float [B,H,n_qc,D], cent_k float [B,H,n_kc,D] (device).
 * topk      1 <= topk <= n_kc; n_kc <= 8192.
 * blocks    out int32 [B,H,n_qc,topk]: for each query cluster, the indices of
 *           the topk key clusters with the largest score qbar . kbar (ties to
 *           the lower index), in ascending order.
 * scores    out float [B,H,n_qc,n_kc] or NULL: the fp32 score matrix.
 */
int ca_route(const float* cent_q, const float* cent_k, int B, int H, int n_qc, int n_kc,
             int D, int topk, int32_t* blocks, float* scores, void* ws, size_t ws_bytes,
             void* stream);

/*
 * ca_route_noalloc -- ca_route for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same centroid scores and top-k selection as ca_route with
 * scores = NULL, bit for bit, but the score matrix lives in a scratch array
 * inside the library instead of a caller workspace, so neither the caller
 * nor the library allocates anything.
 *
 * Arguments as ca_route (cent_q, cent_k, B, H, n_qc, n_kc, D, topk, blocks,
 * stream); the stream's device must be the current device.
 * Limit: B*H*n_qc*n_kc <= 8388608 scores (32 MiB of fp32; e.g. 40 heads of
 * 256 x 256 clusters, or 8 heads of 1024 x 1024); larger calls return
 * CA_ERR_UNSUPPORTED before launching anything (use ca_route).
 * The scratch is one device array per GPU, held from the first call on that
 * GPU until the process ends and shared by every call on it: calls that
 * overlap on one GPU (concurrent streams or threads) race on it and must be
 * serialised by the caller. Nothing in it needs to start at zero (every
 * score is written before it is read). CA_ERR_HIP if the array's device
 * address cannot be obtained.
 */
int ca_route_noalloc(const float* cent_q, const float* cent_k, int B, int H, int n_qc, int n_kc,
                     int D, int topk, int32_t* blocks, void* stream);

/*
 * ca_route_adaptive -- centroid scoring and adaptive selection (v1 §3.3.2
 * "Selection"; later revision §4.2): for each query cluster, the key
 * clusters of highest score until both min_count clusters and a fraction
 * `recall` of the estimated attention mass are selected.
 *
 * The estimated mass of key cluster j for query cluster a is
 * n_j exp(tau (s_aj - max_j s_aj)), every member taken at the centroid logit
 * (the term that stands for an excluded cluster in Eq. 21). The cutoff is
 * found by two histogram passes with shared edges for the two criteria:
 * 128 bins spanning the row's lowest to highest score, then 128 sub-bins of
 * the lower of the two cutoff bins; every cluster at or above the lower
 * edge of the lower cutoff sub-bin is selected, so at least min_count
 * clusters are taken and their estimated mass reaches recall x total. A
 * score's bin is formed in fp32: key = min(16383, floor(((s - lo) * (128 /
 * (hi - lo))) * 128)), bin key >> 7, sub-bin key & 127; masses are summed
 * exactly as integers in units of 2^-40; the target is floor(recall x total).
 * All clusters are taken when a row's scores are all equal or
 * n_kc <= min_count.
 *
 * cent_q    float [B,H,n_qc,D], cent_k float [B,H,n_kc,D] (device).
 * counts_k  int32 [B,H,n_kc]: key cluster sizes n_j (ca_cluster's counts).
 * scale     tau of the mass estimate; 0 means 1/sqrt(D).
 * recall    in [0, 1] (0: a pure count criterion).
 * min_count >= 1 (16 in the pages' adaptive setting).
 * blocks    out int32 [B,H,n_qc,n_kc]: row a holds its nsel[a] selected key
 *           clusters in ascending order, then -1 up to n_kc.
 * nsel      out int32 [B,H,n_qc]: the number selected.
 * scores    out float [B,H,n_qc,n_kc] or NULL (then the workspace holds it;
 *           its size is that of CA_OP_ROUTE).
 * Errors as ca_route; CA_ERR_INVALID_ARG for recall outside [0, 1],
 * min_count < 1, a negative or non-finite scale.
 */
int ca_route_adaptive(const float* cent_q, const float* cent_k, const int32_t* counts_k, int B,
                      int H, int n_qc, int n_kc, int D, float scale, float recall, int min_count,
                      int32_t* blocks, int32_t* nsel, float* scores, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * ca_attend -- block-sparse attention over the selected clusters with
 * optional striped mean-compensation (v1 §1.2 Eq. 2 and Eq. 5-6; App. A
 * Eq. 21-22; v1 §3.1 on the padded remainder cluster).
 *
 * Q, K, V   [B,H,N,D] of type dt (device, read only).
 * perm_q, perm_k  int32 [B,H,N]: cluster-major permutations as produced by
 *           ca_cluster (any permutation is accepted: e.g. random clusters).
 * blocks    int32 [B,H,n_c,topk]: selected key clusters per query cluster,
 *           each in [0, n_c), distinct within a row (as produced by ca_route).
 * compensate  nonzero: every key cluster not selected by a query's cluster
 *           enters the query's softmax once, with logit scale*q.kbar_c +
 *           ln n_c and value vbar_c (centroids of the original K and V rows).
 * scale     softmax temperature; 0 means 1/sqrt(D). With compensate a
 *           positive scale must be at least 1e-30 (the centroid term is
 *           carried as ln n_c / scale inside the score accumulation).
 * O         out [B,H,N,D] of type dt, original token order.
 * lse       out float [B,H,N] or NULL: natural log of the softmax denominator
 *           (the "attention denominator" of v1 §3.1) including the running
 *           maximum, i.e. log sum over the attended terms of exp(logit).
 */
int ca_attend(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H, int N,
              int D, const int32_t* perm_q, const int32_t* perm_k, int cluster_size,
              const int32_t* blocks, int topk, int compensate, float scale, void* O,
              float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * ca_attend_var -- ca_attend with a variable number of selected clusters per
 * query cluster (the output of ca_route_adaptive; v1 §3.3.2).
 *
 * blocks    int32 [B,H,n_c,max_sel]: row a holds nsel[a] distinct key
 *           clusters in [0, n_c); entries past nsel[a] are not read.
 * nsel      int32 [B,H,n_c] (device): 1 <= nsel[a] <= max_sel (values
 *           outside [0, max_sel] are clamped to it).
 * max_sel   row stride of blocks, 1 <= max_sel <= n_c.
 * Every other argument, the workspace (CA_OP_ATTEND) and the errors are
 * those of ca_attend; CA_ERR_INVALID_ARG also for a null nsel.
 */
int ca_attend_var(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H, int N,
                  int D, const int32_t* perm_q, const int32_t* perm_k, int cluster_size,
                  const int32_t* blocks, const int32_t* nsel, int max_sel, int compensate,
                  float scale, void* O, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * ca_attend_ex -- ca_attend with query clusters of size cluster_size_q and key
 * clusters of size cluster_size_k (the pages pair 64-token query clusters with
 * 128-token key clusters, v1 §3.1), an optional variable selection and
 * shared key/value heads.
 *
 * kv_heads  0 or H: K and V are [B,H,N,D]. Else K and V are [B,kv_heads,N,D]
 *           with kv_heads dividing H, and query head h reads the rows of head
 *           h / (H / kv_heads) (grouped- or multi-query attention; perm_k and
 *           blocks stay per query head, as ca_cluster with the same kv_heads
 *           produces them). CA_ERR_INVALID_ARG if kv_heads does not divide H.
 * kv_shared 0, or 1 when perm_k's rows are identical within each group of
 *           H / kv_heads query heads (ca_cluster with kv_share = 1 produces
 *           that; v1 §6.2 "Extension beyond MHA"): the cluster-major key and
 *           value tiles and the centroids are then built once per group, from
 *           the group's first head, and every head of the group reads them.
 *           The output is that of kv_shared = 0 on the same inputs.
 *           CA_ERR_INVALID_ARG for other values.
 * perm_q    int32 [B,H,N], clusters of cluster_size_q (n_qc = ceil(N/c_q)).
 * perm_k    int32 [B,H,N], clusters of cluster_size_k (n_kc = ceil(N/c_k)).
 * cluster_size_q <= cluster_size_k, both in {64, 128, 256}.
 * blocks    int32 [B,H,n_qc,max_sel]: key clusters in [0, n_kc) per query
 *           cluster; with nsel, row a holds nsel[a] of them.
 * nsel      int32 [B,H,n_qc] (device) or NULL (every row holds max_sel).
 * max_sel   1 <= max_sel <= n_kc.
 * Workspace: CA_OP_ATTEND with cluster_size = cluster_size_k. Other
 * arguments and errors as ca_attend; CA_ERR_UNSUPPORTED for a query cluster
 * size above the key cluster size.
 */
int ca_attend_ex(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H,
                 int kv_heads, int kv_shared, int N, int D, const int32_t* perm_q, const int32_t* perm_k,
                 int cluster_size_q, int cluster_size_k, const int32_t* blocks,
                 const int32_t* nsel, int max_sel, int compensate, float scale, void* O,
                 float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * FP8 attention (dtype CA_BF16_FP8 in ca_attend, ca_attend_var, ca_attend_ex
 * and ca_dense). The pages' kernel is quantized and is compared with
 * quantized dense attention (v1 §4.1 "Baselines"); the scheme is not given
 * there, so this one is stated: each query row is one group, the keys of a
 * cluster form groups of 64 consecutive members of its permutation (a short
 * cluster's last group holds its valid members; ca_dense: 64 consecutive
 * tokens), and with compensation the key centroids, rounded to bf16, form
 * groups of 64 consecutive clusters. A group is quantized as by
 * ca_quantize_e4m3; the logit is scale * s_q * s_k * sum(code_q * code_k)
 * accumulated in fp32. Values, P.V and the output are as with CA_BF16. The
 * workspace is that of CA_BF16.
 *
 * With CA_BF16_FP8_PV the P.V product runs on FP8 operands as well (the
 * pages compare "given equal quantization", v1 §4.1; the scheme is again
 * stated here). Values are grouped per head dimension over 32 consecutive
 * members of a key cluster (ca_dense: 32 consecutive tokens; compensation:
 * 32 consecutive value centroids rounded to bf16); a group shares the scale
 * 2^e, e the smallest integer with max|v| <= 448 * 2^e (at least -127, 0 for
 * an all-zero group), codes e4m3(v * 2^-e) rounded to nearest even (the OCP
 * microscaling E8M0 block scale, applied by the matrix core). The attention
 * weights exp(logit - m) against the kernel's running maximum m (at most
 * 2^8) are rounded to e4m3 before the product; the denominator sums them in
 * fp32 before that rounding. Query clusters must be 128 or 256
 * (CA_ERR_UNSUPPORTED otherwise). The workspace is that of CA_BF16.
 */

/*
 * ca_quantize_e4m3 -- rows to FP8 (OCP E4M3) codes, one scale per group of
 * `group` consecutive rows (the last group may be short): amax = max |x| over
 * the group, inv = fp32(448 / amax) (0 for an all-zero group), code =
 * e4m3(fp32(x * inv)) rounded to nearest even (sign kept, so -0 gives 0x80),
 * scale = fp32(amax / 448); x is recovered as code value * scale. The
 * attention's FP8 operands are made by the same device code.
 *
 * X       [rows, D] of type dt (CA_BF16 or CA_F32; device, read only).
 * codes   out uint8 [rows, D] (device).
 * scales  out float [ceil(rows / group)] (device).
 * Errors: CA_ERR_INVALID_ARG for null pointers, another dtype, rows, D or
 * group < 1, rows * D or group * D >= 2^31. Inputs must be finite.
 */
int ca_quantize_e4m3(const void* X, ca_dtype dt, int64_t rows, int D, int group, uint8_t* codes,
                     float* scales, void* stream);

/*
 * ca_dense -- dense attention baseline, o_i = sum_j softmax_j(scale q_i.k_j) v_j
 * (v1 §1.2 Eq. 1). Same layouts and conventions as ca_attend.
 */
int ca_dense(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H, int N,
             int D, float scale, void* O, float* lse, void* ws, size_t ws_bytes,
             void* stream);

/*
 * Profiling hook. When start and stop are non-NULL hipEvent_t handles,
 * subsequent ca_attend and ca_dense calls made by the calling thread record
 * `start` on their stream immediately before their main attention kernel and
 * `stop` immediately after it, so the caller can time that kernel alone with
 * hipEventElapsedTime. Pass NULL, NULL to switch it off. Returns CA_OK.
 * This is per-thread state outside the stateless contract above: while it is
 * set, ca_attend* and ca_dense enqueue the two event records besides their
 * kernels (their results are unchanged). It is off by default.
 */
int ca_profile_events(void* start, void* stop);

/*
 * Peak-rate probe (a measurement utility beside the path, not part of it).
 * kind 0: `blocks` workgroups of 4 waves each issue 4 x iters independent
 *         v_mfma_f32_32x32x16_bf16 (32768 FLOP each) from registers.
 * kind 1: `blocks` workgroups of 4 waves each issue 8 x iters conflict-free
 *         ds_read_b128 (1 KB per wave instruction) from LDS.
 * out: device float [blocks * 4], written with a checksum per wave.
 * The caller times the call with events on `stream`. Returns
 * CA_ERR_INVALID_ARG for a bad kind, blocks outside [1, 65535], iters < 1 or
 * a null out.
 */
int ca_peak_probe(int kind, int blocks, int iters, float* out, void* stream);

/* Static description of a status code. */
const char* ca_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* ca_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CLUSTERATTN_CA_H */
