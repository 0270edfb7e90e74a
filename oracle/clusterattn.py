"""CPU oracle for ClusterAttention's forward path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the bench's CPU-baseline leg
may import this module. The HIP product path never imports, links or calls it,
and it shares no code, tables or constants with the HIP sources.

It is a plain, slow fp64 NumPy implementation of what the method computes,
written step by step from the paper "ClusterAttention: A training-free speedup
of bidirectional attention" (arXiv 2608.26965; cited below as "v1" for the
arXiv HTML of version 1 and "rev" for the later revision's text). Inputs are
the exact values the GPU sees (bf16-rounded numbers widened to fp64).

Where the paper leaves a step open, the reading taken here is stated at the
function that implements it. Summary of those readings:

* splitting variant: basic recursive splitting (PDDP) with the attention
  metric injected into the power iteration (v1 §3.2.1 "Basic recursive
  splitting"; v1 §6.1 notes the metric can be injected so no
  eigendecomposition is needed); optionally the diagonalized variant (v1
  §3.2.1 "Diagonalized recursive splitting", rev §4.1.1): the vectors are
  rotated once into the principal-component basis of the whole set (in the
  transform's geometry, z = R x) and each node splits along the coordinate
  of highest sample variance; basis columns are ordered by descending
  eigenvalue, each with its largest-magnitude entry made positive;
* the subsample of min(a d, |S|) vectors is a Bernoulli sample at rate
  min(1, a d / |S|) decided by a 64-bit content hash of each token's raw
  input bits (so it is deterministic, identical on CPU and GPU, and
  independent of token order); fewer than 2 sampled rows -> the whole node;
* principal component of the centred sample covariance; p power iterations
  (default 8), warm start = normalise(parent estimate + unit random vector),
  random vector = Irwin-Hall(4) normals from a splitmix64 stream;
* split threshold at the multiple of c closest to |S|/2 (equidistant ->
  the smaller); values equal at the threshold go left in token-id order;
* top-k selection is exact with ties to the lower key-cluster index;
* striped mean-compensation is per query, with the cluster's valid count as
  weight and the original (untransformed) key and value centroids;
* the optional FP8 Q.K^T operands (OCP E4M3): queries quantized per token,
  keys per 64 consecutive members of a cluster (per 64 consecutive tokens in
  dense attention), compensation centroids rounded to bf16 and quantized per
  64 consecutive clusters; scale amax / 448, codes rounded to nearest even
  from fp32(x * fp32(448 / amax)); values stay exact.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, library routines, published generator
outputs or brute force (the query and key representations and the whole
clustering against textbook PDDP on explicitly transformed vectors, the warm
start against its geometric characterisation), except ``cluster_agreement``
(a reporting helper).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15          # splitmix64 increment (Steele, Lea, Flood 2014)
MIX1 = 0xBF58476D1CE4E5B9            # splitmix64 finaliser multipliers
MIX2 = 0x94D049BB133111EB

DOMAIN_SAMPLE = 0x53   # salt domains of the two random draws of the method
DOMAIN_WARM = 0x57

TENSOR_Q = 0
TENSOR_K = 1


# ---------------------------------------------------------------------------
# Counter-based random numbers: splitmix64 (Steele, Lea & Flood, "Fast
# splittable pseudorandom number generators", OOPSLA 2014).
# ---------------------------------------------------------------------------

def fmix64(z):
    """splitmix64 output finaliser on Python ints or uint64 numpy arrays."""
    if isinstance(z, (int, np.integer)) and not isinstance(z, np.ndarray):
        z = int(z) & MASK64
        z = ((z ^ (z >> 30)) * MIX1) & MASK64
        z = ((z ^ (z >> 27)) * MIX2) & MASK64
        return z ^ (z >> 31)
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        return z ^ (z >> np.uint64(31))


def splitmix64_stream(seed: int, count: int) -> list[int]:
    """The first ``count`` outputs of splitmix64 seeded with ``seed``."""
    out, s = [], seed & MASK64
    for _ in range(count):
        s = (s + GOLDEN) & MASK64
        out.append(fmix64(s))
    return out


def chain(*vals: int) -> int:
    """Fold small integers into one 64-bit key: z <- fmix64((z ^ v) + golden)."""
    z = 0
    for v in vals:
        z = fmix64(((z ^ (int(v) & MASK64)) + GOLDEN) & MASK64)
    return z


def row_hash(words: np.ndarray) -> np.ndarray:
    """64-bit content hash of each row of 32-bit words, shape [N, W] -> [N].

    A polynomial hash over Z/2^64 finished by the splitmix64 finaliser:
    h = fmix64( sum_j w_j golden^(j+1)  mod 2^64 ).
    """
    words = np.asarray(words, dtype=np.uint64)
    pw = np.array([pow(GOLDEN, j + 1, 1 << 64) for j in range(words.shape[1])], dtype=np.uint64)
    with np.errstate(over="ignore"):
        s = (words * pw[None, :]).sum(axis=1, dtype=np.uint64)
    return fmix64(s)


def row_words(X: np.ndarray, dtype: str) -> np.ndarray:
    """The raw 32-bit words of each token row as stored on the device.

    bf16 rows: word j packs elements 2j (low half) and 2j+1 (high half);
    fp32 rows: word j is the bit pattern of element j.
    """
    X32 = np.ascontiguousarray(X, dtype=np.float32)
    u = X32.view(np.uint32)
    if dtype == "f32":
        return u.astype(np.uint64)
    if dtype != "bf16":
        raise ValueError(dtype)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not exact bfloat16")
    b = (u >> np.uint32(16)).astype(np.uint64)
    return b[:, 0::2] | (b[:, 1::2] << np.uint64(16))


def warm_vector(seed: int, head: int, tensor: int, level: int, node: int, d: int) -> np.ndarray:
    """Random normal-like vector for the power-iteration warm start.

    Component j takes the (j+1)-th output of a splitmix64 stream keyed by
    (seed, head, tensor, level, node); its four 16-bit fields f_0..f_3 give an
    Irwin-Hall(4) variate sum_k (f_k + 1/2)/65536 - 2 (mean 0, variance 1/3;
    the scale is irrelevant because the vector is normalised).
    """
    base = chain(seed, DOMAIN_WARM, head, tensor, level, node)
    r = np.empty(d, np.float64)
    for j, z in enumerate(splitmix64_stream(base, d)):
        s = 0.0
        for k in range(4):
            s += (((z >> (16 * k)) & 0xFFFF) + 0.5) / 65536.0
        r[j] = s - 2.0
    return r


# ---------------------------------------------------------------------------
# Tree layout (v1 §3.1 and §3.2.1; rev §4.1.1)
# ---------------------------------------------------------------------------

def split_size(n: int, c: int) -> int:
    """Left-child size of a node with n > c members.

    The split leaves the multiple of c closest to n/2 below the threshold
    (v1 §3.2.1): t = j c with j >= 1 and t < n; when two multiples are equally
    close (n an odd multiple of c) the smaller one is taken.
    """
    if n <= c:
        raise ValueError("a node of size <= c is a leaf")
    best = None
    for j in range(1, (n - 1) // c + 1):
        t = j * c
        if best is None or abs(2 * t - n) < abs(2 * best - n):
            best = t
    return best


@dataclass
class Node:
    level: int
    index: int      # position of the node among the 2^level slots of its level
    off: int
    n: int


def tree_levels(N: int, c: int) -> list[list[Node]]:
    """Nodes of the recursive split, grouped by depth.

    The layout depends only on N and c. A node with n > c members splits into
    [off, off+t) and [off+t, off+n), t = split_size(n, c); nodes with n <= c are
    leaves (v1 §3.1: at most one cluster differs from c, the one that absorbs
    the remainder). Children of slot j are slots 2j and 2j+1.
    """
    levels: list[list[Node]] = []
    cur = [Node(0, 0, 0, N)]
    while cur:
        levels.append(cur)
        nxt = []
        for nd in cur:
            if nd.n > c:
                t = split_size(nd.n, c)
                nxt.append(Node(nd.level + 1, 2 * nd.index, nd.off, t))
                nxt.append(Node(nd.level + 1, 2 * nd.index + 1, nd.off + t, nd.n - t))
        cur = nxt
    return levels


def leaf_sizes(N: int, c: int) -> list[int]:
    """Cluster sizes in leaf order (left first)."""
    out = []

    def rec(n):
        if n <= c:
            out.append(n)
            return
        t = split_size(n, c)
        rec(t)
        rec(n - t)
    rec(N)
    return out


# ---------------------------------------------------------------------------
# Transforms (v1 §3.2.2, Eq. 12-16; App. B Eq. 37-47; App. C Eq. 48-49)
# ---------------------------------------------------------------------------

def metric_matrices(Q: np.ndarray, K: np.ndarray):
    """M_q = Q^T Q / n (Eq. 12), key mean, M_k = K_c^T K_c / n (Eq. 15)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    n = Q.shape[0]
    Mq = Q.T @ Q / n
    kbar = K.mean(axis=0)
    Kc = K - kbar
    Mk = Kc.T @ Kc / K.shape[0]
    return Mq, Mk, kbar


def root_matrix(M: np.ndarray) -> np.ndarray:
    """Symmetric PSD root of a metric matrix via eigendecomposition, negative
    eigenvalues clamped to zero (v1 §3.2.2 "Key clustering")."""
    w, V = np.linalg.eigh(M)
    w = np.clip(w, 0.0, None)
    return (V * np.sqrt(w)) @ V.T


def query_normalisers(Q: np.ndarray, G: np.ndarray) -> np.ndarray:
    """s_i = (q_i^T G q_i)^{-1/2}, so that s_i q_i represents R q / |R q| with
    R^T R = G (Eq. 16 / Eq. 47). A query with q^T G q <= 0 gets s_i = 0."""
    Q = np.asarray(Q, np.float64)
    v = np.einsum("ij,jk,ik->i", Q, G, Q)
    s = np.zeros_like(v)
    pos = v > 0
    s[pos] = 1.0 / np.sqrt(v[pos])
    return s


# ---------------------------------------------------------------------------
# Recursive splitting (v1 §3.2.1 "Basic recursive splitting"; rev §4.1.1)
# ---------------------------------------------------------------------------

@dataclass
class ClusterOpts:
    transform: bool = True          # attention-aware metrics (v1 §3.2.2)
    query_normalize: bool = True    # top-k query representation (Eq. 16)
    power_iters: int = 8            # p
    sample_factor: int = 1          # a
    seed: int = 0
    split_mode: str = "power"       # "power" (basic) or "diag" (diagonalized)


def sample_threshold(n: int, d: int, a: int) -> int:
    """Integer acceptance threshold floor(2^32 min(1, a d / n))."""
    if a * d >= n:
        return 1 << 32
    return ((a * d) << 32) // n


def sample_members(members: np.ndarray, hashes: np.ndarray, level: int, tensor: int,
                   d: int, a: int, seed: int) -> np.ndarray:
    """The node's subsample (reading: Bernoulli at rate min(1, a d / n) on a
    content hash; fewer than two rows -> the whole node)."""
    n = members.shape[0]
    thr = sample_threshold(n, d, a)
    salt = chain(seed, DOMAIN_SAMPLE, tensor, level)
    top = fmix64(hashes[members] ^ np.uint64(salt)) >> np.uint64(32)
    T = members[top.astype(np.uint64) < np.uint64(thr)] if thr < (1 << 32) else members
    if T.shape[0] < 2:
        T = members
    return T


def warm_start(seed: int, head: int, tensor: int, level: int, index: int, d: int,
               parent: np.ndarray | None) -> np.ndarray:
    """Start vector of the power iteration at node (level, index) (v1 §3.2.1
    "Basic recursive splitting": the estimate starts from the parent's
    principal-component estimate averaged with a random normal vector of about
    the same norm). Read as u0 = normalise(u_parent + r / |r|), u_parent the
    parent's unit direction; at the root (no parent) u0 = r / |r|. r is
    warm_vector of the node; if the sum vanishes, r / |r| is kept."""
    r = warm_vector(seed, head, tensor, level, index, d)
    r = r / np.linalg.norm(r)
    if parent is None:
        return r
    s = parent + r
    ns = np.linalg.norm(s)
    return s / ns if ns > 0 else r


def principal_direction(Xs: np.ndarray, M: np.ndarray, u0: np.ndarray, p: int) -> np.ndarray:
    """p power iterations u <- M C u / |M C u| from u0, C the centred sample
    covariance. With M = R^T R this is the power iteration on R C R^T written
    for u = R^T v, so u . x = v . (R x): the metric is injected and no root
    matrix is formed. If an iterate vanishes the warm start is kept."""
    Xs = np.asarray(Xs, np.float64)
    xbar = Xs.mean(axis=0)
    Xc = Xs - xbar
    C = Xc.T @ Xc / Xs.shape[0]
    u = u0.copy()
    for _ in range(p):
        w = M @ (C @ u)
        nrm = math.sqrt(float(w @ w))
        if nrm == 0.0:
            return u0.copy()
        u = w / nrm
    return u


def pc_basis(X: np.ndarray, M: np.ndarray):
    """Principal-component basis of the whole set in the geometry M (v1
    §3.2.1 "Diagonalized recursive splitting"; rev §4.1.1).

    The vectors are represented as z = R x with R the root matrix of M (the
    transforms of v1 §3.2.2); C is the centred covariance of the z over all
    rows and C = W diag(lam) W^T its eigendecomposition. Returns A = R W and
    lam: coordinate j of a vector is y_j = x . a_j (a_j column j of A).
    Columns are ordered by descending eigenvalue; each column a_j of A is
    signed so that its largest-magnitude entry is positive (the first such
    entry on ties), which fixes which child is "left" at a split. The
    coordinates do not depend on which root of M is used (any F with
    F F^T = M gives the same a_j up to sign), so the sign is fixed on A
    itself.
    """
    X = np.asarray(X, np.float64)
    R = root_matrix(M)
    Z = X @ R
    Zc = Z - Z.mean(axis=0)
    C = Zc.T @ Zc / X.shape[0]
    lam, W = np.linalg.eigh(C)
    order = np.argsort(-lam, kind="stable")
    lam, W = lam[order], W[:, order]
    A = R @ W
    for j in range(A.shape[1]):
        k = int(np.argmax(np.abs(A[:, j])))
        if A[k, j] < 0:
            A[:, j] = -A[:, j]
    return A, lam


def diag_direction(Xs: np.ndarray, A: np.ndarray):
    """Coordinate of highest variance over the sample rows Xs (population
    variance of y_j = x . a_j; the lowest index on ties) and its column of A:
    splitting along y_j is projecting onto a_j."""
    Y = np.asarray(Xs, np.float64) @ A
    var = ((Y - Y.mean(axis=0)) ** 2).mean(axis=0)
    j = int(np.argmax(var))
    return j, A[:, j].copy()


def split_by_scores(members: np.ndarray, scores: np.ndarray, t: int):
    """Members ordered by (score, token id); the first t go left. Both halves
    keep the node's order (ascending token id). Scores that compare equal
    (including -0.0 and +0.0) are ordered by token id."""
    scores = np.asarray(scores, np.float64) + 0.0   # -0.0 -> +0.0
    order = np.lexsort((members, scores))
    left_pos = np.sort(order[:t])
    mask = np.zeros(members.shape[0], bool)
    mask[left_pos] = True
    return members[mask], members[~mask]


@dataclass
class TreeTrace:
    """Per-level state of one clustering tree (for stage-isolated checks)."""
    perms: list = field(default_factory=list)    # perm before level l (and final)
    scores: list = field(default_factory=list)   # projection per position at level l
    dirs: dict = field(default_factory=dict)     # (level, index) -> u


def cluster_tree(X: np.ndarray, M: np.ndarray, hashes: np.ndarray, c: int, opts: ClusterOpts,
                 head: int, tensor: int, trace: TreeTrace | None = None,
                 basis: np.ndarray | None = None) -> np.ndarray:
    """Recursive PDDP splitting of the rows of X under geometry M.

    Returns perm with perm[p] = token at cluster-major position p; cluster j
    occupies [j c, j c + n_j). At each node: subsample, centred covariance,
    warm-started power iteration with the metric injected, projection of all
    members, split at the multiple of c closest to half. With
    opts.split_mode == "diag" the direction is instead the basis column of
    highest sample variance (``basis`` = A of pc_basis, computed here if not
    given).
    """
    X = np.asarray(X, np.float64)
    N, d = X.shape
    perm = np.arange(N, dtype=np.int64)
    parent_dir: dict = {}
    diag = opts.split_mode == "diag"
    if diag and basis is None:
        basis, _ = pc_basis(X, M)
    for level, nodes in enumerate(tree_levels(N, c)):
        if not any(nd.n > c for nd in nodes):
            break
        new = perm.copy()
        sc = np.full(N, np.nan)
        for nd in nodes:
            if nd.n <= c:
                continue
            members = perm[nd.off:nd.off + nd.n]
            T = sample_members(members, hashes, level, tensor, d, opts.sample_factor, opts.seed)
            if diag:
                _, u = diag_direction(X[T], basis)
            else:
                par = parent_dir.get((level - 1, nd.index // 2))
                u0 = warm_start(opts.seed, head, tensor, level, nd.index, d, par)
                u = principal_direction(X[T], M, u0, opts.power_iters)
            parent_dir[(level, nd.index)] = u
            scores = X[members] @ u
            sc[nd.off:nd.off + nd.n] = scores
            t = split_size(nd.n, c)
            left, right = split_by_scores(members, scores, t)
            new[nd.off:nd.off + t] = left
            new[nd.off + t:nd.off + nd.n] = right
        if trace is not None:
            trace.perms.append(perm.copy())
            trace.scores.append(sc)
        perm = new
    if trace is not None:
        trace.perms.append(perm.copy())
        trace.dirs = parent_dir
    return perm


def head_representations(Q: np.ndarray, K: np.ndarray, opts: ClusterOpts):
    """Vectors and geometry to split for one head.

    Keys: x = k under M_q (Eq. 11-14). Queries: x = s q under M_k with
    s = (q^T M_k q)^{-1/2} (Eq. 15-16, Eq. 47). Without the transform both
    geometries are the identity.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    d = Q.shape[1]
    if opts.transform:
        Mq, Mk, _ = metric_matrices(Q, K)
    else:
        Mq = Mk = np.eye(d)
    s = query_normalisers(Q, Mk) if opts.query_normalize else np.ones(Q.shape[0])
    return s[:, None] * Q, Mk, K, Mq


def cluster(Q: np.ndarray, K: np.ndarray, c: int, opts: ClusterOpts | None = None,
            dtype: str = "bf16", traces: dict | None = None, c_k: int | None = None,
            key_share: int = 1):
    """Cluster queries and keys of every (batch, head) separately (v1 §3.1).

    Q, K: [B, H, N, D]. Returns perm_q, perm_k of shape [B, H, N] (int64).
    The flattened head index b*H + h keys the random draws. The keys' tree
    uses cluster size c_k when given (v1 §3.1 pairs 64-token query clusters
    with 128-token key clusters), else c. key_share = g > 1: the heads form
    groups of g consecutive query heads over one key/value head (K holds
    that head's rows repeated per query head), and each group's keys are
    clustered once, under the mean of the group's query metrics (v1 §6.2
    "Extension beyond MHA", its first option), with the random draws of the
    group's first head; every head of the group gets that permutation.
    """
    opts = opts or ClusterOpts()
    B, H, N, D = Q.shape
    pq = np.empty((B, H, N), np.int64)
    pk = np.empty((B, H, N), np.int64)
    for b in range(B):
        for h in range(H):
            head = b * H + h
            Xq, Gq, Xk, Gk = head_representations(Q[b, h], K[b, h], opts)
            hq = row_hash(row_words(Q[b, h], dtype))
            hk = row_hash(row_words(K[b, h], dtype))
            tq = TreeTrace() if traces is not None else None
            tk = TreeTrace() if traces is not None else None
            pq[b, h] = cluster_tree(Xq, Gq, hq, c, opts, head, TENSOR_Q, tq)
            if traces is not None:
                traces[(b, h, TENSOR_Q)] = tq
            if key_share > 1:
                if h % key_share:
                    lead = h - h % key_share
                    pk[b, h] = pk[b, lead]
                    if traces is not None:        # the group's one key tree
                        traces[(b, h, TENSOR_K)] = traces[(b, lead, TENSOR_K)]
                    continue
                Gk = np.mean([head_representations(Q[b, h + i], K[b, h + i], opts)[3]
                              for i in range(key_share)], axis=0)
            pk[b, h] = cluster_tree(Xk, Gk, hk, c_k or c, opts, head, TENSOR_K, tk)
            if traces is not None:
                traces[(b, h, TENSOR_K)] = tk
    return pq, pk


# ---------------------------------------------------------------------------
# Centroids and assignment (v1 §3.3, Eq. 18-20; rev §4.2)
# ---------------------------------------------------------------------------

def centroids(X: np.ndarray, perm: np.ndarray, c: int):
    """Means of the original vectors over each cluster's valid members, and
    the member counts. X: [N, D], perm: [N]. Returns ([n_c, D], [n_c])."""
    X = np.asarray(X, np.float64)
    sizes = leaf_sizes(X.shape[0], c)
    cent = np.empty((len(sizes), X.shape[1]))
    for j, nj in enumerate(sizes):
        cent[j] = X[perm[j * c:j * c + nj]].mean(axis=0)
    return cent, np.asarray(sizes, np.int64)


def cluster_scores(cq: np.ndarray, ck: np.ndarray) -> np.ndarray:
    """A[a, j] = qbar_a . kbar_j: the mean logit between the clusters (Eq. 18;
    the 1/sqrt(d) temperature does not change the ranking)."""
    return np.asarray(cq, np.float64) @ np.asarray(ck, np.float64).T


def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the lower index, ascending."""
    scores = np.asarray(scores, np.float64) + 0.0
    idx = np.arange(scores.shape[0])
    order = np.lexsort((idx, -scores))
    return np.sort(order[:k])


def route(cq: np.ndarray, ck: np.ndarray, k: int, scores: np.ndarray | None = None) -> np.ndarray:
    """Top-k key clusters per query cluster (v1 §3.3.2). cq: [n_qc, D],
    ck: [n_kc, D] (or a given score matrix). Returns [n_qc, k] ascending."""
    A = cluster_scores(cq, ck) if scores is None else np.asarray(scores, np.float64)
    return np.stack([topk_row(A[a], k) for a in range(A.shape[0])])


def cluster_masses(scores: np.ndarray, counts: np.ndarray, tau: float) -> np.ndarray:
    """Estimated attention mass of each key cluster for one query cluster:
    every member of cluster c taken at the centroid logit, n_c exp(tau s_c)
    (the same term that stands for an excluded cluster in Eq. 21), relative
    to the largest score so that nothing overflows."""
    s = np.asarray(scores, np.float64)
    return np.asarray(counts, np.float64) * np.exp(tau * (s - s.max()))


def adaptive_row(scores: np.ndarray, counts: np.ndarray, tau: float, recall: float,
                 min_count: int, nbins: int = 128) -> np.ndarray:
    """Adaptive selection for one query cluster (v1 §3.3.2 "Selection"; later
    revision §4.2): the key clusters of highest centroid score until both an
    estimated attention-mass recall and a minimum count are reached, found by
    two histogram passes with shared edges for the two criteria.

    Pass 1: n_bins bins spanning the lowest to the highest score; scanning
    from the top bin, the cutoff bin of each criterion is the first at which
    the cumulative count (mass) reaches min_count (recall x total mass); the
    lower of the two is refined. Pass 2: n_bins sub-bins within it, the same
    scan with the totals of the bins above carried in; the final cutoff is the
    lower edge of the lower of the two cutoff sub-bins, and every cluster at
    or above it is selected. Returns the selected indices, ascending.

    The bin of a score decides membership, so it is computed in fp32 exactly
    as the kernel does: u = (s - lo) * (n_bins / (hi - lo)), key =
    min(n_bins^2 - 1, floor(u * n_bins)); coarse bin key // n_bins, sub-bin
    key % n_bins. Masses are fp64, summed exactly as integers in units of
    2^-40 (every mass is at most n_c <= 2^13, so sums fit in 62 bits); the
    mass target is floor(recall * total) in fp64. All clusters are selected
    when the scores are all equal or there are at most min_count clusters.
    """
    s32 = np.asarray(scores, np.float32)
    n = s32.shape[0]
    if n <= min_count:
        return np.arange(n)
    lo, hi = s32.min(), s32.max()
    if not hi > lo:
        return np.arange(n)
    scale = np.float32(nbins) / (hi - lo)
    u = (s32 - lo) * scale
    key = np.minimum(nbins * nbins - 1, np.floor(u * np.float32(nbins)).astype(np.int64))
    coarse, fine = key // nbins, key % nbins
    mass = [int(v) for v in np.rint(cluster_masses(s32.astype(np.float64), counts, tau) * 2.0**40)]
    total = sum(mass)
    target = int(math.floor(recall * float(total)))
    ones = [1] * n

    def cutoff(members, bins, weights, carried, thr):
        # highest bin b with carried + sum over bins >= b of weights >= thr
        # (n_bins when the carried total already reaches it, 0 if none does)
        if carried >= thr:
            return nbins
        hist = [0] * nbins
        for i in members:
            hist[bins[i]] += weights[i]
        cum = carried
        for b in range(nbins - 1, -1, -1):
            cum += hist[b]
            if cum >= thr:
                return b
        return 0

    everyone = range(n)
    b_star = min(cutoff(everyone, coarse, ones, 0, min_count),
                 cutoff(everyone, coarse, mass, 0, target))
    above = [i for i in everyone if coarse[i] > b_star]
    inb = [i for i in everyone if coarse[i] == b_star]
    f_c = cutoff(inb, fine, ones, len(above), min_count)
    f_m = cutoff(inb, fine, mass, sum(mass[i] for i in above), target)
    k_star = b_star * nbins + min(f_c, f_m)
    return np.flatnonzero(key >= k_star)


def route_adaptive(cq: np.ndarray, ck: np.ndarray, counts: np.ndarray, tau: float, recall: float,
                   min_count: int = 16, scores: np.ndarray | None = None):
    """Adaptive selection per query cluster: a list of ascending index
    arrays (their lengths vary)."""
    A = cluster_scores(cq, ck) if scores is None else np.asarray(scores, np.float64)
    return [adaptive_row(A[a], counts, tau, recall, min_count) for a in range(A.shape[0])]


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) operands of the Q.K^T product. The pages run a quantized
# block-sparse kernel and compare it with quantized dense attention "given
# equal quantization" (v1 §4.1 "Baselines"; rev §5 "Experiments" and §4
# "Method" on the kernel); they do not give the scheme. Reading taken here:
# queries are quantized per token, keys per block of 64 consecutive keys of a
# cluster's member list (the kernel's key sub-tile), compensation centroids
# per block of 64 consecutive clusters after rounding to bf16 (the precision
# in which centroids are streamed); each group has scale amax / 448 and
# codes e4m3(x * (448 / amax)), both computed in fp32; P.V stays exact.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3
    mantissa bits; subnormals at exponent field 0; S.1111.111 is NaN; no
    infinities; largest finite 448)."""
    c = np.asarray(codes, np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E == 0, M / 8.0 * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), finite values
    of magnitude >= 464 saturate to +-448, NaN gives 0x7F; the sign of zero
    is kept. The spacing in binade [2^e, 2^(e+1)) is 2^(e-3), and 2^-9 below
    2^-6 (the subnormals)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                          # a = m 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)                   # binade, floored at the subnormals
    q = np.exp2(e - 3.0)
    n = np.rint(a / q)                           # round half to even
    v = np.minimum(n * q, E4M3_MAX)
    _, ev = np.frexp(v)
    Ev = ev - 1
    normal = v >= 2.0 ** -6
    mant = np.where(normal, v / np.exp2(Ev) * 8.0 - 8.0, 0.0)
    code = np.where(normal, ((Ev + 7) << 3) + mant, v / 2.0 ** -9).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def bf16_nearest(x) -> np.ndarray:
    """fp32 values rounded to bfloat16 (round to nearest, ties to even on the
    fp32 bit pattern), returned as fp32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32)


def quantize_e4m3(X, group: int):
    """Rows of X in groups of `group` consecutive rows (the last group may be
    short), one scale per group: amax = max |x| over the group, inv =
    fp32(448 / amax) (0 for an all-zero group), code = e4m3(fp32(x * inv)),
    scale = fp32(amax / 448). X holds fp32 values. Returns (codes uint8 like
    X, scales float32 [ceil(rows / group)])."""
    X = np.asarray(X, np.float32)
    R = X.shape[0]
    ng = (R + group - 1) // group
    codes = np.empty(X.shape, np.uint8)
    scales = np.empty(ng, np.float32)
    for g in range(ng):
        blk = X[g * group:(g + 1) * group]
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        inv = np.float32(E4M3_MAX) / amax if amax > 0 else np.float32(0)
        codes[g * group:(g + 1) * group] = e4m3_encode(blk * np.float32(inv))
        scales[g] = amax / np.float32(E4M3_MAX)
    return codes, scales


def dequantize_e4m3(codes, scales, group: int) -> np.ndarray:
    """code value x group scale, exact in fp64."""
    rows = np.arange(codes.shape[0]) // group
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[rows][:, None]


def fp8_rows(X, group: int) -> np.ndarray:
    """X after quantization in row groups and dequantization."""
    return dequantize_e4m3(*quantize_e4m3(X, group), group)


def fp8_keys(K, perm_k, ck: int, tile: int = 64) -> np.ndarray:
    """K (token order) after quantization per block of `tile` consecutive
    members of each key cluster's member list (a short cluster's last block
    holds only its valid members)."""
    K = np.asarray(K, np.float32)
    out = np.empty(K.shape, np.float64)
    for j, nj in enumerate(leaf_sizes(K.shape[0], ck)):
        mem = np.asarray(perm_k[j * ck:j * ck + nj])
        for p in range(0, nj, tile):
            rows = mem[p:p + tile]
            out[rows] = fp8_rows(K[rows], len(rows))
    return out


def fp8_centroids(kbar, tile: int = 64) -> np.ndarray:
    """Key centroids rounded to bf16, then quantized per block of `tile`
    consecutive clusters."""
    return fp8_rows(bf16_nearest(kbar), tile)


# FP8 (OCP E4M3) value operands of the P.V product (reading, as for Q.K^T:
# the pages give no scheme). Values are grouped per head dimension over 32
# consecutive members of a key cluster's member list (32 consecutive tokens in
# dense attention, 32 consecutive key centroids after rounding to bf16 for
# compensation), and a group shares a power-of-two scale 2^e: the block scale
# of the OCP microscaling formats (an E8M0 exponent per 32 elements), with e
# the smallest integer such that amax <= 448 * 2^e (e >= -127; e = 0 for an
# all-zero group), codes e4m3(x * 2^-e). The attention weights P multiply
# these dequantized values; P itself is kept exact here (the kernel rounds P
# to E4M3 against its running maximum, so the tests bound that rounding
# instead of reproducing it).

def e8m0_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, at least -127; 0 when
    amax == 0. With amax = m 2^x (m in [0.5, 1)) and 448 = 0.875 2^9:
    e = x - 9 if m <= 0.875 else x - 8."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, x = math.frexp(amax)
    return max(-127, x - 9 if m <= 0.875 else x - 8)


def quantize_mx_e4m3(X, block: int):
    """Columns of X in groups of `block` consecutive rows (the last group may
    be short), one power-of-two scale per (group, column): returns codes
    (uint8, like X) and exponents (int64 [ceil(rows / block), columns])."""
    X = np.asarray(X, np.float64)
    R, D = X.shape
    ng = (R + block - 1) // block
    codes = np.empty(X.shape, np.uint8)
    expo = np.zeros((ng, D), np.int64)
    for g in range(ng):
        blk = X[g * block:(g + 1) * block]
        for d in range(D):
            e = e8m0_exponent(np.max(np.abs(blk[:, d])) if blk.size else 0.0)
            expo[g, d] = e
            codes[g * block:(g + 1) * block, d] = e4m3_encode(blk[:, d] * 2.0 ** -e)
    return codes, expo


def fp8_value_rows(X, block: int) -> np.ndarray:
    """X after quantize_mx_e4m3 and dequantization (exact in fp64)."""
    codes, expo = quantize_mx_e4m3(X, block)
    rows = np.arange(codes.shape[0]) // block
    return e4m3_decode(codes) * np.exp2(expo[rows].astype(np.float64))


def fp8_values(V, perm_k, ck: int, block: int = 32) -> np.ndarray:
    """V (token order) after quantization per dimension over each block of
    `block` consecutive members of a key cluster's member list (a short
    cluster's last block holds only its valid members)."""
    V = np.asarray(V, np.float64)
    out = np.empty(V.shape, np.float64)
    for j, nj in enumerate(leaf_sizes(V.shape[0], ck)):
        mem = np.asarray(perm_k[j * ck:j * ck + nj])
        for p in range(0, nj, block):
            rows = mem[p:p + block]
            out[rows] = fp8_value_rows(V[rows], len(rows))
    return out


def fp8_value_centroids(vbar, block: int = 32) -> np.ndarray:
    """Value centroids rounded to bf16, then quantized per dimension over
    blocks of `block` consecutive clusters."""
    return fp8_value_rows(bf16_nearest(vbar).astype(np.float64), block)


# ---------------------------------------------------------------------------
# Attention (v1 §1.2 Eq. 1-2; App. A Eq. 21-22)
# ---------------------------------------------------------------------------

def _softmax_combine(logits: np.ndarray, values: np.ndarray):
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ values) / l
    return o, (m + np.log(l))[:, 0]


def dense_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float | None = None,
                    qk: str = "exact", pv: str = "exact"):
    """o_i = sum_j softmax_j(tau q_i . k_j) v_j and LSE_i = log sum_j exp(.)
    for one head (Eq. 1). Q, K, V: [N, D]. qk="e4m3": the logits use the FP8
    operands (queries per token, keys per block of 64 consecutive tokens).
    pv="e4m3": the values are the FP8 ones (per dimension over blocks of 32
    consecutive tokens); the weights stay exact."""
    tau = 1.0 / math.sqrt(np.shape(Q)[1]) if not scale else float(scale)
    if qk == "e4m3":
        Q, K = fp8_rows(Q, 1), fp8_keys(K, np.arange(np.shape(K)[0]), 64)
    if pv == "e4m3":
        V = fp8_values(V, np.arange(np.shape(V)[0]), np.shape(V)[0])
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    return _softmax_combine(tau * (Q @ K.T), V)


def attention_terms(Q, K, V, perm_q, perm_k, c: int, blocks, compensate: bool,
                    scale: float | None = None, clusters=None, c_k: int | None = None,
                    qk: str = "exact", pv: str = "exact"):
    """The terms sparse_attention combines, per query cluster a: yields
    (a, query tokens, logits [n_a, terms], values [terms, D]). Query i of
    cluster a has one term per key of the selected clusters Sel(a), logit
    tau q_i . k_j and value v_j (Eq. 2), and with compensation one term per
    excluded key cluster, logit tau q_i . kbar_c + ln|c| and value vbar_c
    (Eq. 21-22, the centroid weight counted |c| times)."""
    N, D = np.shape(Q)
    tau = 1.0 / math.sqrt(D) if not scale else float(scale)
    ck = c_k or c
    qs = leaf_sizes(N, c)
    ks = leaf_sizes(np.shape(K)[0], ck)
    kbar, cnt = centroids(K, perm_k, ck)
    vbar, _ = centroids(V, perm_k, ck)
    if qk == "e4m3":
        Q, K, kbar = fp8_rows(Q, 1), fp8_keys(K, perm_k, ck), fp8_centroids(kbar)
    if pv == "e4m3":
        V, vbar = fp8_values(V, perm_k, ck), fp8_value_centroids(vbar)
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    for a in (range(len(qs)) if clusters is None else clusters):
        na = qs[a]
        qi = perm_q[a * c:a * c + na]
        sel = np.asarray(blocks[a], np.int64)
        keys = np.concatenate([perm_k[j * ck:j * ck + ks[j]] for j in sel])
        logits = tau * (Q[qi] @ K[keys].T)
        vals = V[keys]
        if compensate:
            mask = np.ones(len(ks), bool)
            mask[sel] = False
            ex = np.nonzero(mask)[0]
            if ex.size:
                cl = tau * (Q[qi] @ kbar[ex].T) + np.log(cnt[ex].astype(np.float64))[None, :]
                logits = np.concatenate([logits, cl], axis=1)
                vals = np.concatenate([vals, vbar[ex]], axis=0)
        yield a, qi, logits, vals


def sparse_attention(Q, K, V, perm_q, perm_k, c: int, blocks, compensate: bool,
                     scale: float | None = None, clusters=None, c_k: int | None = None,
                     qk: str = "exact", pv: str = "exact"):
    """Block-sparse attention of one head with optional striped
    mean-compensation.

    Query i of cluster a attends with token resolution to every key of the
    selected clusters Sel(a) (Eq. 2). With compensation, every excluded key
    cluster enters once through its centroid: logit tau q_i . kbar_c +
    ln|c| and value vbar_c, which is Eq. 21-22 (the centroid weight w_c
    counted |c| times); attention_terms lists these terms. Returns O in
    original token order and LSE. ``clusters`` restricts the work to those
    query clusters (the rows of the other queries are NaN). Key clusters have
    size c_k when given, else c.
    qk="e4m3": the logits use the FP8 operands (fp8_rows per query, fp8_keys,
    fp8_centroids); the values and the centroid values stay exact unless
    pv="e4m3" (fp8_values, fp8_value_centroids; the weights stay exact).
    """
    N = np.shape(Q)[0]
    O = np.full((N, np.shape(V)[1]), np.nan)
    L = np.full(N, np.nan)
    for _, qi, logits, vals in attention_terms(Q, K, V, perm_q, perm_k, c, blocks, compensate,
                                               scale, clusters, c_k, qk, pv):
        o, lse = _softmax_combine(logits, vals)
        O[qi] = o
        L[qi] = lse
    return O, L


def attend(Q, K, V, perm_q, perm_k, c: int, blocks, compensate: bool, scale=None, c_k=None,
           qk: str = "exact", pv: str = "exact"):
    """sparse_attention over every (batch, head): Q,K,V [B,H,N,D]."""
    B, H, N, D = Q.shape
    O = np.empty((B, H, N, V.shape[-1]))
    L = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = sparse_attention(Q[b, h], K[b, h], V[b, h], perm_q[b, h],
                                                perm_k[b, h], c, blocks[b][h], compensate, scale,
                                                c_k=c_k, qk=qk, pv=pv)
    return O, L


def dense(Q, K, V, scale=None, qk: str = "exact", pv: str = "exact"):
    """dense_attention over every (batch, head)."""
    B, H, N, D = Q.shape
    O = np.empty((B, H, N, V.shape[-1]))
    L = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = dense_attention(Q[b, h], K[b, h], V[b, h], scale, qk, pv)
    return O, L


def forward(Q, K, V, c: int, topk: int, compensate: bool = True, opts: ClusterOpts | None = None,
            dtype: str = "bf16", scale=None, qk: str = "exact", pv: str = "exact"):
    """The whole path: cluster -> centroids -> route -> attend (v1 §1.1)."""
    pq, pk = cluster(Q, K, c, opts, dtype)
    B, H, N, D = Q.shape
    blocks = np.empty((B, H, len(leaf_sizes(N, c)), topk), np.int64)
    for b in range(B):
        for h in range(H):
            cq, _ = centroids(Q[b, h], pq[b, h], c)
            ck, _ = centroids(K[b, h], pk[b, h], c)
            blocks[b, h] = route(cq, ck, topk)
    O, L = attend(Q, K, V, pq, pk, c, blocks, compensate, scale, qk=qk, pv=pv)
    return O, L, pq, pk, blocks


# ---------------------------------------------------------------------------
# Reporting helper
# ---------------------------------------------------------------------------

def cluster_agreement(perm_a: np.ndarray, perm_b: np.ndarray, c: int) -> float:
    """Fraction of tokens whose cluster id is the same under two perms."""
    N = perm_a.shape[-1]
    ida = np.empty(N, np.int64); idb = np.empty(N, np.int64)
    ida[perm_a] = np.arange(N) // c
    idb[perm_b] = np.arange(N) // c
    return float(np.mean(ida == idb))
