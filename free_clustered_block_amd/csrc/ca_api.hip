// Host side of the C ABI declared in include/ca.h: argument validation,
// workspace layout and launch sequencing. No call allocates memory or
// synchronises with the device; ca_cluster creates its side stream (one per
// GPU) and its fork/join events (per host thread and GPU) once, at first use.
#include <cmath>
#include <mutex>
#include <string>

#include "ca.h"
#include "kernels.h"

namespace ca {

static thread_local std::string g_last_error;
static thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
void set_error(const std::string& s) { g_last_error = s; }

namespace {

constexpr size_t kAlign = 256;

// Carves typed, 256-byte aligned sub-buffers out of the workspace. With a null
// base it only measures, so sizing and carving share one layout.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t size() const { return (off + kAlign - 1) / kAlign * kAlign; }
};

struct ClusterWs {
  float* partial;
  uint64_t* hash;      // by token (= by position before the first split)
  uint64_t* hashB;     // by position, ping-pong with hash
  float *Mq, *Mk, *kbar, *Mpk;
  uint16_t* gsplit;
  float* s;
  int32_t *permA, *permB;
  uint32_t* keys;
  float *dirA, *dirB;
  int32_t* sample;
  int32_t* chunk_cnt;
  int32_t* stok;
  float* zbuf;
  float *Cq, *Rbuf, *Zbuf, *At;   // diagonalized splitting: basis of each tree
  uint16_t* At3;                  // its three-term bf16 split
  int32_t* jsel;                  // chosen coordinate per node
  float* Y;                       // coordinates of every vector (diagonalized only)
  int32_t* wide;                  // wide split of the large-node levels (or null)
};

ClusterWs plan_cluster(Carver& cv, int BH, int N, int D, int c, bool diag) {
  ClusterWs w;
  const size_t T = 2 * (size_t)BH;
  const int rows = metric_rows_per_chunk(N, BH);
  const size_t nchunks = (N + rows - 1) / rows;
  const int L = tree_levels_host(N, c);
  const size_t slots = L > 0 ? ((size_t)1 << (L - 1)) : 1;
  w.partial = cv.take<float>((size_t)BH * nchunks * (2 * (size_t)D * D + D));
  w.hash = cv.take<uint64_t>(T * N);
  w.hashB = cv.take<uint64_t>(T * N);
  w.Mq = cv.take<float>((size_t)BH * D * D);
  w.Mk = cv.take<float>((size_t)BH * D * D);
  w.kbar = cv.take<float>((size_t)BH * D);
  w.Mpk = cv.take<float>(T * D * D);
  w.gsplit = cv.take<uint16_t>((size_t)BH * 3 * D * D);
  w.s = cv.take<float>((size_t)BH * N);
  w.permA = cv.take<int32_t>(T * N);
  w.permB = cv.take<int32_t>(T * N);
  w.keys = cv.take<uint32_t>(T * N);
  w.dirA = cv.take<float>(T * slots * D);
  w.dirB = cv.take<float>(T * slots * D);
  w.sample = cv.take<int32_t>(T * N);
  w.chunk_cnt = cv.take<int32_t>(T * ((N + c - 1) / c));
  w.stok = cv.take<int32_t>(T * N);
  w.zbuf = cv.take<float>(T * N);
  w.Cq = cv.take<float>((size_t)BH * D * D);
  w.Rbuf = cv.take<float>(T * D * D);
  w.Zbuf = cv.take<float>(T * D * D);
  w.At = cv.take<float>(T * D * D);
  w.At3 = cv.take<uint16_t>(T * 3 * D * D);
  w.jsel = cv.take<int32_t>(T * slots);
  w.Y = diag ? cv.take<float>(T * N * D) : nullptr;
  const size_t ww = wide_split_words(BH, N, c);
  w.wide = ww ? cv.take<int32_t>(ww) : nullptr;
  return w;
}

void plan_attend(Carver& cv, AttnArgs& a, bool with_tiles) {
  const size_t BH = a.BH, nc = a.nc, ncp = attn_ncp(a.nc), D = a.D, c = a.c;
  if (with_tiles) {
    a.kc = cv.take<uint16_t>(BH * nc * c * D);
    a.vt = cv.take<uint16_t>(BH * nc * c * D);
    a.kbar_hi = cv.take<uint16_t>(BH * ncp * D);
    a.vbar_t = cv.take<uint16_t>(BH * ncp * D);
  } else {
    a.kc = a.vt = a.kbar_hi = a.vbar_t = nullptr;
  }
  a.logn = cv.take<float>(BH * ncp);
  a.kbar32 = cv.take<float>(BH * ncp * D);
  a.vbar32 = cv.take<float>(BH * ncp * D);
  if (a.dtype == 3 && with_tiles) {
    // FP8 values: the value sub-tiles take the bf16 value tiles' region (half
    // its size and the scales), the centroid sub-tiles the fp32 value
    // centroids past the key-centroid scales
    a.vt8 = reinterpret_cast<uint8_t*>(a.vt);
    a.vbar8 = reinterpret_cast<uint8_t*>(a.vbar32) + (BH * (ncp / 64) * 4 + 255) / 256 * 256;
  }
  if (a.dtype >= 2 && with_tiles) {
    // FP8 keys: the codes take the first half of the bf16 key tiles and the
    // sub-tile scales the second; the centroid codes and scales take the
    // fp32 centroid arrays, which only the fp32 path uses
    a.kc8 = reinterpret_cast<uint8_t*>(a.kc);
    a.kscale = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.kc) + BH * nc * c * D);
    a.kbar8 = reinterpret_cast<uint8_t*>(a.kbar32);
    a.kbscale = a.vbar32;
    a.kc = nullptr;
  }
}

constexpr int kDenseTile = 128;

int attn_dtype(int dt) {
  return dt == CA_BF16 ? 0 : dt == CA_F32 ? 1 : dt == CA_BF16_FP8 ? 2 : 3;
}

bool supported_c(int c) { return c == 64 || c == 128 || c == 256; }
bool supported_d(int d) { return d == 64 || d == 128; }

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return 0;
  if (!ws) return fail(CA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(CA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(CA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                      " bytes, got " + std::to_string(ws_bytes));
  return 0;
}

int after_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return CA_OK;
}

int check_common(int dt, int B, int H, int N, int D, bool fp8_ok = false) {
  if (dt != CA_BF16 && dt != CA_F32 && !(fp8_ok && (dt == CA_BF16_FP8 || dt == CA_BF16_FP8_PV)))
    return fail(CA_ERR_INVALID_ARG, fp8_ok ? "unknown dtype" : "unknown dtype (CA_BF16_FP8 and CA_BF16_FP8_PV are for attention only)");
  if (B < 1 || H < 1 || N < 1 || D < 1) return fail(CA_ERR_INVALID_ARG, "B, H, N, D must be >= 1");
  if ((int64_t)B * H > 32767) return fail(CA_ERR_UNSUPPORTED, "B*H must be <= 32767");
  if ((int64_t)B * H * N >= (int64_t)1 << 31) return fail(CA_ERR_INVALID_ARG, "B*H*N must be < 2^31");
  if (!supported_d(D)) return fail(CA_ERR_UNSUPPORTED, "D must be 64 or 128");
  return 0;
}

// The key trees' split levels run on a side stream beside the query trees':
// at the top levels every direction and split launch is latency-bound and
// fills few CUs, so each tensor's launches overlap the other's projection
// (splitting each tensor's trees over more streams measured no faster). The
// side stream is forked from the caller's stream and joined back to it by
// events, so the call stays ordered on the caller's stream (and a graph
// captured there takes both branches). One side stream per GPU (non-blocking,
// default priority) and one event pair per host thread and GPU, each created
// at its first use and kept until the process ends.
constexpr int kMaxDevices = 64;
int side_stream(hipStream_t* side, hipEvent_t* fork, hipEvent_t* join) {
  int dev = 0;
  CA_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(CA_ERR_UNSUPPORTED, "device index must be < 64");
  static std::mutex mu;
  static hipStream_t streams[kMaxDevices] = {};
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!streams[dev]) CA_HIP_CHECK(hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking));
    *side = streams[dev];
  }
  thread_local hipEvent_t ev[kMaxDevices][2] = {};
  for (int i = 0; i < 2; ++i)
    if (!ev[dev][i]) CA_HIP_CHECK(hipEventCreateWithFlags(&ev[dev][i], hipEventDisableTiming));
  *fork = ev[dev][0];
  *join = ev[dev][1];
  return 0;
}

}  // namespace
}  // namespace ca

using namespace ca;

extern "C" {

int ca_tree_levels(int N, int cluster_size) {
  if (N < 1 || cluster_size < 1) return -1;
  return tree_levels_host(N, cluster_size);
}

size_t ca_workspace_size(ca_op op, int B, int H, int N, int D, int cluster_size, int topk) {
  if (B < 1 || H < 1 || N < 1 || D < 1) return SIZE_MAX;
  const int BH = B * H;
  Carver cv(nullptr);
  switch (op) {
    case CA_OP_CLUSTER:
    case CA_OP_CLUSTER_DIAG:
      if (cluster_size < 1 || N < cluster_size) return SIZE_MAX;
      plan_cluster(cv, BH, N, D, cluster_size, op == CA_OP_CLUSTER_DIAG);
      return cv.size();
    case CA_OP_ROUTE: {
      // N = n_qc and cluster_size = n_kc for this op
      const size_t nq = N, nk = cluster_size;
      (void)cv.take<float>((size_t)BH * nq * nk);
      return cv.size();
    }
    case CA_OP_ATTEND: {
      if (cluster_size < 1 || N < cluster_size) return SIZE_MAX;
      AttnArgs a{};
      a.BH = BH; a.N = N; a.D = D; a.c = cluster_size; a.nc = (N + cluster_size - 1) / cluster_size;
      plan_attend(cv, a, true);
      return cv.size();
    }
    case CA_OP_DENSE: {
      AttnArgs a{};
      a.BH = BH; a.N = N; a.D = D; a.c = kDenseTile; a.nc = (N + kDenseTile - 1) / kDenseTile;
      plan_attend(cv, a, true);
      return cv.size();
    }
  }
  (void)topk;
  return SIZE_MAX;
}

int ca_cluster(const void* Q, const void* K, ca_dtype dt, int B, int H, int N, int D,
               int cluster_size, const ca_cluster_opts* opts, int32_t* perm_q, int32_t* perm_k,
               float* cent_q, float* cent_k, int32_t* counts, void* ws, size_t ws_bytes,
               void* stream) {
  set_error("");
  if (!Q || !K || !perm_q || !perm_k || !cent_q || !cent_k)
    return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  if (int e = check_common(dt, B, H, N, D)) return e;
  const int c = cluster_size;
  if (!supported_c(c)) return fail(CA_ERR_UNSUPPORTED, "cluster_size must be 64, 128 or 256");
  if (N < c) return fail(CA_ERR_INVALID_ARG, "N must be >= cluster_size");
  if ((N + c - 1) / c > 8192) return fail(CA_ERR_UNSUPPORTED, "at most 8192 clusters");
  ca_cluster_opts o = {1, 1, 8, 1, 0, nullptr, nullptr, nullptr, 0, nullptr, 0, 0, 0};
  if (opts) o = *opts;
  const int kvh = o.kv_heads ? o.kv_heads : H;   // key/value heads
  if (kvh < 1 || kvh > H || H % kvh != 0)
    return fail(CA_ERR_INVALID_ARG, "kv_heads must be 0 or divide H");
  const int kvg = H / kvh;
  if (o.kv_share != 0 && o.kv_share != 1) return fail(CA_ERR_INVALID_ARG, "kv_share must be 0 or 1");
  const int kshare = o.kv_share ? kvg : 1;   // query heads per shared key tree
  const int ck = o.cluster_size_k ? o.cluster_size_k : c;   // key cluster size
  if (!supported_c(ck)) return fail(CA_ERR_UNSUPPORTED, "cluster_size_k must be 0, 64, 128 or 256");
  if (N < ck) return fail(CA_ERR_INVALID_ARG, "N must be >= cluster_size_k");
  if (ck != c && (o.trace_perm || o.trace_score || o.trace_dir))
    return fail(CA_ERR_UNSUPPORTED, "traces need equal query and key cluster sizes");
  if (o.split_mode != 0 && o.split_mode != 1)
    return fail(CA_ERR_INVALID_ARG, "split_mode must be 0 (power iteration) or 1 (diagonalized)");
  if (o.power_iters < 1 || o.power_iters > 1000)
    return fail(CA_ERR_INVALID_ARG, "power_iters must be in [1, 1000]");
  if (o.sample_factor < 1 || o.sample_factor > 4096)
    return fail(CA_ERR_INVALID_ARG, "sample_factor must be in [1, 4096]");
  if ((2 * B * H) > 65535) return fail(CA_ERR_UNSUPPORTED, "2*B*H must be <= 65535");
  const int BH = B * H;
  Carver cv(ws);
  ClusterWs w = plan_cluster(cv, BH, N, D, c < ck ? c : ck, o.split_mode == 1);
  if (int e = check_ws(ws, ws_bytes, cv.size())) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t TN = 2 * (size_t)BH * N;

  const int dti = dt == CA_BF16 ? 0 : 1;
  launch_metric(Q, K, dti, BH, N, D, o.transform, w.partial, w.hash, w.Mq, w.Mk, w.kbar, w.gsplit,
                w.Mpk, kvg, st);
  if (kshare > 1) launch_pool_key_metric(w.Mq, w.Mpk, BH, D, kshare, st);
  // the query normalisers: before the basis (which weights the queries by
  // them), else on the query trees' stream only (the key trees do not read them)
  auto qnorm = [&] {
    launch_qnorm(Q, dti, BH, N, D, o.transform, o.query_normalize, w.gsplit, w.Mk, w.s, st);
  };
  if (o.split_mode == 1) {
    qnorm();
    launch_basis(Q, dt == CA_BF16 ? 0 : 1, BH, N, D, o.transform, w.s, w.Mq, w.Mk, w.partial, w.Cq,
                 w.Rbuf, w.Zbuf, w.At, st);
    if (o.trace_basis)
      CA_HIP_CHECK(hipMemcpyAsync(o.trace_basis, w.At, 2 * (size_t)BH * D * D * 4,
                                  hipMemcpyDeviceToDevice, st));
    launch_rotate(Q, K, dt == CA_BF16 ? 0 : 1, BH, N, D, w.s, w.At, w.At3, w.Y, kvg, st);
  }
  launch_perm_init(w.permA, 2 * BH, N, st);
  // the split levels of one tensor's trees (rows base, base + step, ...) with
  // cluster size ct, enqueued on stream rs; returns the permutation array
  // that holds their final order in `fin`
  // per-tree row strides of the level buffers, the same for every level and
  // both tensors (the workspace's sizes, from the smaller cluster size)
  const int cmin = c < ck ? c : ck;
  const int nch_all = (N + cmin - 1) / cmin;
  const int lmax = tree_levels_host(N, cmin);
  const int node_slots = lmax > 0 ? 1 << (lmax - 1) : 1;
  auto run_levels = [&](int ct, int step, int base, int32_t*& fin, hipStream_t rs) -> int {
    const int L = tree_levels_host(N, ct);
    int32_t* cur = w.permA;
    int32_t* nxt = w.permB;
    uint64_t* hcur = w.hash;
    uint64_t* hnxt = w.hashB;
    // trace copies of this run's trees only (rows base, base + step, ...)
    const int ntrees = (2 * BH - base + step - 1) / step;
    auto trace_copy = [&](int32_t* dst, const int32_t* src) -> int {
      CA_HIP_CHECK(hipMemcpy2DAsync(dst + (size_t)base * N, (size_t)step * N * 4, src + (size_t)base * N,
                                    (size_t)step * N * 4, (size_t)N * 4, ntrees,
                                    hipMemcpyDeviceToDevice, rs));
      return 0;
    };
    for (int level = 0; level < L; ++level) {
      if (o.trace_perm)
        if (int e = trace_copy(o.trace_perm + level * TN, cur)) return e;
      LevelArgs a{};
      a.Q = Q; a.K = K; a.dtype = dt == CA_BF16 ? 0 : 1;
      a.BH = BH; a.N = N; a.D = D; a.c = ct; a.level = level; a.kvg = kvg;
      a.transform = o.transform; a.power_iters = o.power_iters; a.sample_factor = o.sample_factor;
      a.split_mode = o.split_mode; a.basis = w.At; a.Y = w.Y; a.jsel = w.jsel;
      a.tree_step = step; a.tree_base = base;
      a.seed = o.seed;
      a.perm_in = cur; a.perm_out = nxt;
      a.hpos_in = hcur; a.hpos_out = hnxt; a.s = w.s; a.Mq = w.Mq; a.Mk = w.Mk; a.Mpk = w.Mpk;
      a.dir_prev = (level & 1) ? w.dirA : w.dirB;
      a.dir_cur = (level & 1) ? w.dirB : w.dirA;
      a.nchunks = nch_all;
      a.node_slots = node_slots;
      a.sample_buf = w.sample; a.chunk_cnt = w.chunk_cnt; a.zbuf_tok = w.stok;
      a.zbuf = w.zbuf; a.keys = w.keys; a.wide = w.wide;
      a.trace_score = o.trace_score ? o.trace_score + level * TN : nullptr;
      a.trace_slots = L > 0 ? (1 << (L - 1)) : 1;
      a.trace_dir = o.trace_dir ? o.trace_dir + (size_t)level * 2 * BH * a.trace_slots * D : nullptr;
      launch_level(a, rs);
      int32_t* t = cur; cur = nxt; nxt = t;
      uint64_t* th = hcur; hcur = hnxt; hnxt = th;
    }
    if (o.trace_perm)
      if (int e = trace_copy(o.trace_perm + (size_t)L * TN, cur)) return e;
    fin = cur;
    return 0;
  };
  // query trees on the caller's stream; beside them the key trees (of the
  // first head of each group when the key clustering is shared) on the side
  // stream. The two touch disjoint rows of every per-tree buffer; each ends
  // with its own permutation output and centroids.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  if (int e = side_stream(&side, &ev_fork, &ev_join)) return e;
  CA_HIP_CHECK(hipEventRecord(ev_fork, st));
  CA_HIP_CHECK(hipStreamWaitEvent(side, ev_fork, 0));
  int32_t *fin_q = nullptr, *fin_k = nullptr;
  int err = 0;
  if (o.split_mode == 0) qnorm();
  if (int e = run_levels(c, 2, 0, fin_q, st)) {
    err = e;
  } else {
    launch_perm_out(fin_q, 0, BH, N, kshare, perm_q, st);
    launch_centroids(Q, K, dti, BH, N, D, c, ck, perm_q, perm_k, cent_q, cent_k, counts, kvg, 0, 1, st);
  }
  if (!err) {
    if (int e = run_levels(ck, 2 * kshare, 1, fin_k, side)) {
      err = e;
    } else {
      launch_perm_out(fin_k, 1, BH, N, kshare, perm_k, side);
      launch_centroids(Q, K, dti, BH, N, D, c, ck, perm_q, perm_k, cent_q, cent_k, counts, kvg, 1, 1,
                       side);
    }
  }
  // join even after a failed enqueue, so the side stream never runs ahead
  CA_HIP_CHECK(hipEventRecord(ev_join, side));
  CA_HIP_CHECK(hipStreamWaitEvent(st, ev_join, 0));
  if (err) return err;
  return after_launch();
}

int ca_route(const float* cent_q, const float* cent_k, int B, int H, int n_qc, int n_kc, int D,
             int topk, int32_t* blocks, float* scores, void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  if (!cent_q || !cent_k || !blocks) return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  if (B < 1 || H < 1 || n_qc < 1 || n_kc < 1) return fail(CA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!supported_d(D)) return fail(CA_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (topk < 1 || topk > n_kc) return fail(CA_ERR_INVALID_ARG, "topk must be in [1, n_kc]");
  if (n_kc > 8192) return fail(CA_ERR_UNSUPPORTED, "n_kc must be <= 8192");
  if ((int64_t)B * H > 32767 || n_qc > 65535) return fail(CA_ERR_UNSUPPORTED, "too many heads or query clusters");
  const int BH = B * H;
  Carver cv(ws);
  float* sc = scores;
  if (!sc) {
    sc = cv.take<float>((size_t)BH * n_qc * n_kc);
    if (int e = check_ws(ws, ws_bytes, cv.size())) return e;
  }
  launch_route(cent_q, cent_k, BH, n_qc, n_kc, D, topk, sc, blocks, static_cast<hipStream_t>(stream));
  return after_launch();
}

int ca_route_noalloc(const float* cent_q, const float* cent_k, int B, int H, int n_qc, int n_kc,
                     int D, int topk, int32_t* blocks, void* stream) {
  set_error("");
  if (!cent_q || !cent_k || !blocks) return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  if (B < 1 || H < 1 || n_qc < 1 || n_kc < 1) return fail(CA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!supported_d(D)) return fail(CA_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (topk < 1 || topk > n_kc) return fail(CA_ERR_INVALID_ARG, "topk must be in [1, n_kc]");
  if (n_kc > 8192) return fail(CA_ERR_UNSUPPORTED, "n_kc must be <= 8192");
  if ((int64_t)B * H > 32767 || n_qc > 65535) return fail(CA_ERR_UNSUPPORTED, "too many heads or query clusters");
  if ((uint64_t)B * H * n_qc * n_kc > kRouteScratchFloats)
    return fail(CA_ERR_UNSUPPORTED, "B*H*n_qc*n_kc exceeds the " + std::to_string(kRouteScratchFloats) +
                                        " scores (32 MiB) of the allocation-free scratch; use ca_route");
  float* sc = nullptr;
  const char* err = "";
  if (route_scratch(&sc, &err)) return fail(CA_ERR_HIP, std::string("scratch address: ") + err);
  launch_route(cent_q, cent_k, B * H, n_qc, n_kc, D, topk, sc, blocks, static_cast<hipStream_t>(stream));
  return after_launch();
}

int ca_route_adaptive(const float* cent_q, const float* cent_k, const int32_t* counts_k, int B,
                      int H, int n_qc, int n_kc, int D, float scale, float recall, int min_count,
                      int32_t* blocks, int32_t* nsel, float* scores, void* ws, size_t ws_bytes,
                      void* stream) {
  set_error("");
  if (!cent_q || !cent_k || !counts_k || !blocks || !nsel)
    return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  if (B < 1 || H < 1 || n_qc < 1 || n_kc < 1) return fail(CA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!supported_d(D)) return fail(CA_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (!(recall >= 0.0f && recall <= 1.0f)) return fail(CA_ERR_INVALID_ARG, "recall must be in [0, 1]");
  if (min_count < 1) return fail(CA_ERR_INVALID_ARG, "min_count must be >= 1");
  if (!(scale >= 0.0f) || !std::isfinite(scale)) return fail(CA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (n_kc > 8192) return fail(CA_ERR_UNSUPPORTED, "n_kc must be <= 8192");
  if ((int64_t)B * H > 32767 || n_qc > 65535) return fail(CA_ERR_UNSUPPORTED, "too many heads or query clusters");
  const int BH = B * H;
  Carver cv(ws);
  float* sc = scores;
  if (!sc) {
    sc = cv.take<float>((size_t)BH * n_qc * n_kc);
    if (int e = check_ws(ws, ws_bytes, cv.size())) return e;
  }
  const float tau = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  launch_route_adaptive(cent_q, cent_k, counts_k, BH, n_qc, n_kc, D, tau, (double)recall, min_count,
                        sc, blocks, nsel, static_cast<hipStream_t>(stream));
  return after_launch();
}

namespace {
int attend_impl(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H,
                int kv_heads, int kv_shared, int N, int D, const int32_t* perm_q, const int32_t* perm_k,
                int cluster_size_q,
                int cluster_size_k, const int32_t* blocks, const int32_t* nsel, int topk,
                int compensate, float scale, void* O, float* lse, void* ws, size_t ws_bytes,
                void* stream) {
  set_error("");
  if (!Q || !K || !V || !perm_q || !perm_k || !blocks || !O)
    return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  if (int e = check_common(dt, B, H, N, D, true)) return e;
  const int c = cluster_size_k, cq = cluster_size_q;
  if (!supported_c(c) || !supported_c(cq))
    return fail(CA_ERR_UNSUPPORTED, "cluster sizes must be 64, 128 or 256");
  if (cq > c) return fail(CA_ERR_UNSUPPORTED, "the query cluster size must not exceed the key cluster size");
  if (dt == CA_BF16_FP8_PV && cq < 128)
    return fail(CA_ERR_UNSUPPORTED, "CA_BF16_FP8_PV needs query clusters of 128 or 256");
  if (N < c) return fail(CA_ERR_INVALID_ARG, "N must be >= the cluster sizes");
  const int nc = (N + c - 1) / c, nqc = (N + cq - 1) / cq;
  if (nc > 8192) return fail(CA_ERR_UNSUPPORTED, "at most 8192 key clusters");
  if ((int64_t)nqc * B * H > 0x7FFFFFFF / 2) return fail(CA_ERR_UNSUPPORTED, "too many query clusters");
  if (topk < 1 || topk > nc) return fail(CA_ERR_INVALID_ARG, "topk must be in [1, n_kc]");
  if (!(scale >= 0.0f) || !std::isfinite(scale)) return fail(CA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (compensate && scale > 0.0f && scale < 1e-30f)
    return fail(CA_ERR_INVALID_ARG, "with compensation a positive scale must be >= 1e-30");
  if (kv_heads < 1 || kv_heads > H || H % kv_heads != 0)
    return fail(CA_ERR_INVALID_ARG, "kv_heads must divide H");
  if (kv_shared != 0 && kv_shared != 1) return fail(CA_ERR_INVALID_ARG, "kv_shared must be 0 or 1");
  AttnArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.dtype = attn_dtype(dt);
  a.kvg = H / kv_heads;
  a.kshare = kv_shared ? a.kvg : 1;
  a.BH = B * H; a.N = N; a.D = D; a.c = c; a.nc = nc; a.cq = cq; a.nqc = nqc; a.topk = topk;
  a.compensate = compensate ? 1 : 0;
  a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  a.perm_q = perm_q; a.perm_k = perm_k; a.blocks = blocks; a.nsel = nsel; a.O = O; a.lse = lse;
  a.ev_start = g_prof_start; a.ev_stop = g_prof_stop;
  Carver cv(ws);
  plan_attend(cv, a, true);
  if (int e = check_ws(ws, ws_bytes, cv.size())) return e;
  launch_attend(a, static_cast<hipStream_t>(stream));
  return after_launch();
}
}  // namespace

int ca_attend(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H, int N, int D,
              const int32_t* perm_q, const int32_t* perm_k, int cluster_size,
              const int32_t* blocks, int topk, int compensate, float scale, void* O, float* lse,
              void* ws, size_t ws_bytes, void* stream) {
  return attend_impl(Q, K, V, dt, B, H, H, 0, N, D, perm_q, perm_k, cluster_size, cluster_size, blocks,
                     nullptr, topk, compensate, scale, O, lse, ws, ws_bytes, stream);
}

int ca_attend_var(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H, int N,
                  int D, const int32_t* perm_q, const int32_t* perm_k, int cluster_size,
                  const int32_t* blocks, const int32_t* nsel, int max_sel, int compensate,
                  float scale, void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!nsel) {
    set_error("");
    return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  }
  return attend_impl(Q, K, V, dt, B, H, H, 0, N, D, perm_q, perm_k, cluster_size, cluster_size, blocks,
                     nsel, max_sel, compensate, scale, O, lse, ws, ws_bytes, stream);
}

int ca_attend_ex(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H,
                 int kv_heads, int kv_shared, int N, int D, const int32_t* perm_q,
                 const int32_t* perm_k, int cluster_size_q, int cluster_size_k,
                 const int32_t* blocks, const int32_t* nsel, int max_sel, int compensate,
                 float scale, void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  return attend_impl(Q, K, V, dt, B, H, kv_heads ? kv_heads : H, kv_shared, N, D, perm_q, perm_k,
                     cluster_size_q, cluster_size_k, blocks, nsel, max_sel, compensate, scale, O,
                     lse, ws, ws_bytes, stream);
}

int ca_dense(const void* Q, const void* K, const void* V, ca_dtype dt, int B, int H, int N, int D,
             float scale, void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  if (!Q || !K || !V || !O) return fail(CA_ERR_INVALID_ARG, "null tensor pointer");
  if (int e = check_common(dt, B, H, N, D, true)) return e;
  if (!(scale >= 0.0f) || !std::isfinite(scale)) return fail(CA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  AttnArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.dtype = attn_dtype(dt);
  a.BH = B * H; a.N = N; a.D = D; a.c = kDenseTile; a.nc = (N + kDenseTile - 1) / kDenseTile;
  a.cq = a.c; a.nqc = a.nc; a.kvg = 1; a.kshare = 1;
  a.topk = a.nc; a.compensate = 0;
  a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  a.O = O; a.lse = lse;
  a.ev_start = g_prof_start; a.ev_stop = g_prof_stop;
  Carver cv(ws);
  plan_attend(cv, a, true);
  if (int e = check_ws(ws, ws_bytes, cv.size())) return e;
  launch_dense(a, static_cast<hipStream_t>(stream));
  return after_launch();
}

int ca_quantize_e4m3(const void* X, ca_dtype dt, int64_t rows, int D, int group, uint8_t* codes,
                     float* scales, void* stream) {
  set_error("");
  if (!X || !codes || !scales) return fail(CA_ERR_INVALID_ARG, "null pointer");
  if (dt != CA_BF16 && dt != CA_F32) return fail(CA_ERR_INVALID_ARG, "dtype must be CA_BF16 or CA_F32");
  if (rows < 1 || D < 1 || group < 1) return fail(CA_ERR_INVALID_ARG, "rows, D and group must be >= 1");
  if (rows * (int64_t)D >= ((int64_t)1 << 31) || (int64_t)group * D >= ((int64_t)1 << 31))
    return fail(CA_ERR_INVALID_ARG, "rows * D and group * D must be < 2^31");
  launch_quantize_e4m3(X, dt == CA_BF16 ? 0 : 1, rows, D, group, codes, scales,
                       static_cast<hipStream_t>(stream));
  return after_launch();
}

int ca_peak_probe(int kind, int blocks, int iters, float* out, void* stream) {
  if ((kind != 0 && kind != 1) || blocks < 1 || blocks > 65535 || iters < 1 || !out)
    return fail(CA_ERR_INVALID_ARG, "ca_peak_probe: kind must be 0 or 1, blocks in [1, 65535], iters >= 1, out non-null");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0) launch_peak_mfma(blocks, iters, out, st);
  else launch_peak_lds(blocks, iters, out, st);
  CA_HIP_CHECK(hipGetLastError());
  return CA_OK;
}

int ca_profile_events(void* start, void* stop) {
  g_prof_start = (start && stop) ? static_cast<hipEvent_t>(start) : nullptr;
  g_prof_stop = (start && stop) ? static_cast<hipEvent_t>(stop) : nullptr;
  return CA_OK;
}

const char* ca_status_string(int status) {
  switch (status) {
    case CA_OK: return "ok";
    case CA_ERR_INVALID_ARG: return "invalid argument";
    case CA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case CA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ca_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
