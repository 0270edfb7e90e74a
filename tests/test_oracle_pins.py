"""Pins of the CPU oracle against what the paper and mathematics fix.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
an identity, invariant, library routine, brute force or published value; the
tests call them on the oracle as written, and ``test_planted_mistakes`` plants
plausible mistakes into the oracle (on the CPU) and requires a pin to fail.
Paper: "ClusterAttention: A training-free speedup of bidirectional attention"
(arXiv 2608.26965 v1).
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle.clusterattn as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _random_head(seed, N=256, D=16, scale=1.0):
    r = _rng(seed)
    Q = r.standard_normal((N, D)) * scale
    K = r.standard_normal((N, D)) * scale + 0.3 * r.standard_normal(D)
    V = r.standard_normal((N, D))
    return Q, K, V


def _dense_weights(Q, K, tau):
    return scipy.special.softmax(tau * (Q @ K.T), axis=1)


# ---------------------------------------------------------------------------
# Random numbers and hashing (build-defined draws; published generator)
# ---------------------------------------------------------------------------

def check_splitmix64_published():
    vals = [int(l, 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if l.strip() and not l.startswith("#")]
    got = o.splitmix64_stream(0, len(vals))
    assert got == vals, (got, vals)
    arr = o.fmix64(np.array([0x9E3779B97F4A7C15 * (i + 1) & o.MASK64 for i in range(3)],
                            dtype=np.uint64))
    assert [int(x) for x in arr] == vals


def test_splitmix64_published_outputs():
    check_splitmix64_published()


def test_row_words_match_device_layout():
    import torch
    r = _rng(1)
    X = r.standard_normal((5, 8)).astype(np.float32)
    Xb = torch.from_numpy(X).to(torch.bfloat16)
    dev_words = Xb.contiguous().view(torch.int32).numpy().astype(np.uint32)
    got = o.row_words(Xb.float().numpy(), "bf16").astype(np.uint32)
    assert np.array_equal(got, dev_words)
    got32 = o.row_words(X, "f32").astype(np.uint32)
    assert np.array_equal(got32, X.view(np.uint32))


def test_row_hash_properties():
    r = _rng(2)
    W = r.integers(0, 2**32, size=(50, 32), dtype=np.uint64)
    h = o.row_hash(W)
    assert len(set(h.tolist())) == 50
    W2 = W.copy()
    W2[:, [3, 4]] = W2[:, [4, 3]]          # the hash depends on word position
    assert np.all(o.row_hash(W2) != h)
    assert np.array_equal(o.row_hash(W[[7, 7, 3]]), h[[7, 7, 3]])
    # scalar and vector finalisers agree
    for z in W[:5, 0]:
        assert o.fmix64(int(z)) == int(o.fmix64(np.array([z], np.uint64))[0])


def test_warm_vector_statistics():
    vals = np.concatenate([o.warm_vector(5, h, t, l, n, 64)
                           for h in range(4) for t in range(2) for l in range(3) for n in range(4)])
    assert abs(vals.mean()) < 0.02
    assert abs(vals.var() - 1.0 / 3.0) < 0.02
    assert np.all(np.abs(vals) <= 2.0)
    a = o.warm_vector(5, 0, 0, 1, 0, 64)
    b = o.warm_vector(5, 0, 0, 1, 1, 64)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, o.warm_vector(5, 0, 0, 1, 0, 64))


# ---------------------------------------------------------------------------
# Tree layout (v1 §3.1, §3.2.1)
# ---------------------------------------------------------------------------

def check_tree_layout():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "tree_video_32760_c128.txt"))
             if l.strip() and not l.startswith("#")]
    spine = [int(x) for x in lines[0]]
    ncl, last, nlev = (int(x) for x in lines[1])
    levels = o.tree_levels(32760, 128)
    got_spine = [lv[-1].n for lv in levels]
    assert got_spine == spine, got_spine
    sizes = o.leaf_sizes(32760, 128)
    assert len(sizes) == ncl and sizes[-1] == last and all(s == 128 for s in sizes[:-1])
    assert sum(1 for lv in levels if any(nd.n > 128 for nd in lv)) == nlev
    for N, c in [(1024, 64), (65536, 128), (262144, 256), (1000, 64), (3 * 64, 64),
                 (5 * 128, 128), (7 * 64 + 1, 64), (130, 64), (65, 64), (64, 64), (17, 1)]:
        sizes = o.leaf_sizes(N, c)
        assert sum(sizes) == N
        assert len(sizes) == -(-N // c)
        assert all(s == c for s in sizes[:-1]) and 0 < sizes[-1] <= c
        for lv in o.tree_levels(N, c):
            for nd in lv:
                if nd.n > c:
                    t = o.split_size(nd.n, c)
                    cands = [j * c for j in range(1, nd.n) if j * c < nd.n]
                    best = min(abs(x - nd.n / 2) for x in cands)
                    ok = [x for x in cands if abs(x - nd.n / 2) == best]
                    assert t == min(ok), (nd.n, c, t, ok)


def test_tree_layout():
    check_tree_layout()


# ---------------------------------------------------------------------------
# Transforms (v1 §3.2.2, App. B, App. C)
# ---------------------------------------------------------------------------

def check_metrics():
    r = _rng(3)
    n, d = 11, 4
    Q = r.standard_normal((n, d))
    K = r.standard_normal((n, d)) + 2.0
    Mq, Mk, kbar = o.metric_matrices(Q, K)
    # Eq. 10-11: (k1-k2)^T M (k1-k2) is the mean squared logit difference.
    for a, b in [(0, 1), (2, 5), (7, 3)]:
        dk = K[a] - K[b]
        assert math.isclose(dk @ Mq @ dk, np.sum((Q @ K[a] - Q @ K[b]) ** 2) / n, rel_tol=1e-12)
    # Eq. 43-46: D^T D over all ordered key pairs = 2 n K_c^T K_c = 2 n^2 M_k.
    D = np.array([K[a] - K[b] for a in range(n) for b in range(n)])
    assert np.allclose(D.T @ D, 2 * n * n * Mk, rtol=1e-12, atol=1e-10)
    assert np.allclose(kbar, [np.mean(K[:, j]) for j in range(d)])
    # Eq. 39: the entries of K_c q sum to zero for every q.
    q = r.standard_normal(d)
    assert abs(np.sum((K - kbar) @ q)) < 1e-10


def test_metrics_closed_forms():
    check_metrics()


def test_query_representation_shift_invariance():
    # Eq. 36-38: shifts delta with K delta = const * 1 leave the representation.
    r = _rng(4)
    n, d = 40, 5
    e = np.zeros(d); e[2] = 1.0
    K = r.standard_normal((n, d)); K[:, 2] = 1.5            # zero variance along e
    Q = r.standard_normal((n, d))
    Mq, Mk, _ = o.metric_matrices(Q, K)
    assert np.allclose(Mk @ e, 0, atol=1e-12)
    s1 = o.query_normalisers(Q, Mk)
    s2 = o.query_normalisers(Q + 0.7 * e, Mk)
    assert np.allclose(s1, s2, rtol=1e-12)


def check_query_normalisers():
    # Eq. 16/47: s q represents R_k q / |R_k q|, so |R_k (s q)| = 1.
    r = _rng(5)
    Q = r.standard_normal((30, 6))
    K = r.standard_normal((30, 6)) @ np.diag([3, 1, 1, 0.5, 0.1, 0.0]) + 1.0
    _, Mk, _ = o.metric_matrices(Q, K)
    R = o.root_matrix(Mk)
    assert np.allclose(R.T @ R, Mk, atol=1e-12)
    s = o.query_normalisers(Q, Mk)
    assert np.allclose(np.linalg.norm((s[:, None] * Q) @ R.T, axis=1), 1.0, rtol=1e-10)
    assert np.all(o.query_normalisers(np.zeros((2, 6)), Mk) == 0.0)


def test_query_normalisers():
    check_query_normalisers()


def _keys_with_known_covariance(U, sig, kbar):
    """Key rows kbar +- sqrt(d) sig_j u_j (j = 1..d, N = 2d): their mean is
    exactly kbar and their centred second moment is exactly U diag(sig^2) U^T,
    while the uncentred one adds kbar kbar^T."""
    d = len(sig)
    E = np.sqrt(d) * (U * np.asarray(sig)[None, :]).T          # row j: sqrt(d) sig_j u_j
    return np.concatenate([kbar + E, kbar - E]), (U * np.asarray(sig) ** 2) @ U.T


def check_head_representations():
    """The vectors and geometries each tensor is split under (v1 §3.2.2 "Key
    clustering", Eq. 10-14, and "Query clustering", Eq. 15-16): keys are the
    raw key rows under the geometry whose quadratic form on a key difference
    is the mean squared logit difference over the queries; queries are s q
    with s > 0 under the centred key covariance, normalised so that the
    root of that covariance maps each to a unit vector."""
    r = _rng(41)
    d = 6
    U = _orthonormal(r, d, d)
    sig = np.array([3.0, 2.0, 1.5, 1.0, 0.5, 0.25])
    kbar = np.array([4.0, -3.0, 2.5, 1.0, -2.0, 3.5])
    K, Sigma = _keys_with_known_covariance(U, sig, kbar)
    N = K.shape[0]
    Q = r.standard_normal((N, d)) + np.linspace(-2.0, 2.0, d)
    Xq, Gq, Xk, Gk = o.head_representations(Q, K, o.ClusterOpts())
    # query geometry: the centred key covariance built above
    assert np.allclose(Gq, Sigma, rtol=1e-12, atol=1e-12), "query geometry"
    # key geometry: Eq. 10-11 on every pair of keys, brute force over queries
    for a in range(N):
        for b in range(N):
            dk = K[a] - K[b]
            want = np.mean((Q @ K[a] - Q @ K[b]) ** 2)
            assert math.isclose(dk @ Gk @ dk, want, rel_tol=1e-10, abs_tol=1e-10), "key geometry"
    assert np.array_equal(Xk, K), "keys are split untransformed"
    # queries: x_i = s_i q_i with s_i > 0 and |R x_i| = 1 for the known root
    R = (U * sig[None, :]) @ U.T                               # R^T R = Sigma
    ratio = np.einsum("ij,ij->i", Xq, Q) / np.einsum("ij,ij->i", Q, Q)
    assert np.all(ratio > 0)
    assert np.allclose(Xq, ratio[:, None] * Q, rtol=1e-12, atol=1e-14), "queries are scaled q"
    assert np.allclose(np.linalg.norm(Xq @ R.T, axis=1), 1.0, rtol=1e-12), "Eq. 16 normaliser"
    # without the transform: identity geometries, unit-length queries
    Xq0, Gq0, Xk0, Gk0 = o.head_representations(Q, K, o.ClusterOpts(transform=False))
    assert np.array_equal(Gq0, np.eye(d)) and np.array_equal(Gk0, np.eye(d))
    assert np.allclose(np.linalg.norm(Xq0, axis=1), 1.0, rtol=1e-12)
    # without the query normalisation (adaptive mode, v1 §6): raw queries
    Xq1, Gq1, _, _ = o.head_representations(Q, K, o.ClusterOpts(query_normalize=False))
    assert np.array_equal(Xq1, Q) and np.allclose(Gq1, Sigma, rtol=1e-12, atol=1e-12)


def test_head_representations():
    check_head_representations()


def _textbook_pddp(Z, c):
    """Boley's PDDP on explicit vectors: split every node larger than c along
    the top eigenvector (numpy.linalg.eigh) of its members' centred
    covariance, at the median. Returns the leaves as a set of frozensets and
    the largest lambda_2 / lambda_1 met (the power iteration's rate)."""
    leaves, worst = set(), 0.0
    stack = [np.arange(Z.shape[0])]
    while stack:
        m = stack.pop()
        if len(m) <= c:
            leaves.add(frozenset(m.tolist()))
            continue
        Zc = Z[m] - Z[m].mean(0)
        w, V = np.linalg.eigh(Zc.T @ Zc / len(m))
        worst = max(worst, w[-2] / w[-1])
        sc = Z[m] @ V[:, -1]
        order = np.argsort(sc, kind="stable")
        stack += [m[order[:len(m) // 2]], m[order[len(m) // 2:]]]
    return leaves, worst


def check_cluster_matches_textbook_pddp():
    """cluster() run to convergence on the whole node (no subsample) splits
    like textbook PDDP on the explicitly transformed vectors of v1 §3.2.2:
    keys as R_q k (Eq. 14, R_q^T R_q = Q^T Q / N), queries as R_k q / |R_k q|
    (Eq. 16, R_k^T R_k the centred key covariance). N = 4c, so every split is
    at the exact median and the leaves do not depend on the eigenvectors'
    signs; compared as sets of leaves."""
    r = _rng(44)
    N, d, c = 64, 4, 16
    Q = r.standard_normal((N, d)) @ np.diag([3.0, 1.5, 0.8, 0.3]) + 0.5
    K = r.standard_normal((N, d)) @ np.diag([0.4, 2.5, 1.0, 3.0]) - 1.0
    Q4, K4 = Q[None, None], K[None, None]
    pq, pk = o.cluster(Q4, K4, c, o.ClusterOpts(power_iters=400, sample_factor=N, seed=9), "f32")

    def sym_root(S):
        w, V = np.linalg.eigh(S)
        return (V * np.sqrt(np.clip(w, 0, None))) @ V.T

    Rq = sym_root(Q.T @ Q / N)
    Kc = K - K.mean(0)
    Rk = sym_root(Kc.T @ Kc / N)
    zq = Q @ Rk.T
    zq = zq / np.linalg.norm(zq, axis=1, keepdims=True)
    for perm, Z in ((pq[0, 0], zq), (pk[0, 0], K @ Rq.T)):
        want, worst = _textbook_pddp(Z, c)
        assert worst < 0.9, worst           # every node's eigengap makes p = 400 converge
        got = {frozenset(perm[j * c:(j + 1) * c].tolist()) for j in range(N // c)}
        assert got == want


def test_cluster_matches_textbook_pddp():
    check_cluster_matches_textbook_pddp()


# ---------------------------------------------------------------------------
# Principal direction with the metric injected (v1 §3.2.1, §3.2.2, §6.1)
# ---------------------------------------------------------------------------

def check_power_iteration_matches_eigh():
    r = _rng(6)
    d = 6
    A = r.standard_normal((d, d))
    M = A @ np.diag([4, 2, 1, 0.5, 0.2, 0.0]) @ A.T          # PSD, rank deficient
    X = r.standard_normal((80, d)) @ np.diag([3, 2, 1.5, 1, 0.5, 0.2]) @ r.standard_normal((d, d))
    R = o.root_matrix(M)
    Y = X @ R.T                                              # explicit transform R x
    Yc = Y - Y.mean(0)
    w, Vv = np.linalg.eigh(Yc.T @ Yc / len(Y))
    assert w[-1] - w[-2] > 1e-3
    vstar = Vv[:, -1]
    u0 = r.standard_normal(d); u0 /= np.linalg.norm(u0)
    u = o.principal_direction(X, M, u0, 200)
    target = R.T @ vstar
    cos = abs(u @ target) / np.linalg.norm(u) / np.linalg.norm(target)
    assert cos >= 1 - 1e-9, cos
    # the same split as PDDP run explicitly on R x
    sgn = np.sign(u @ target)
    members = np.arange(len(X))
    l1, _ = o.split_by_scores(members, X @ u, 40)
    l2, _ = o.split_by_scores(members, sgn * (Y @ vstar), 40)
    assert np.array_equal(l1, l2)


def test_power_iteration_matches_eigh():
    check_power_iteration_matches_eigh()


def check_warm_start_composition():
    """Warm start of the power iteration (v1 §3.2.1 "Basic recursive
    splitting": the parent's estimate averaged with a random normal vector of
    about the same norm). With no power iterations the traced direction of
    every node is its start: at the root the node's unit random vector, below
    it the bisector of the parent's unit direction and the node's unit random
    vector (unit length, equal cosine to both, in their span)."""
    r = _rng(42)
    N, d, c = 200, 5, 16
    X = r.standard_normal((N, d)) @ r.standard_normal((d, d))
    hashes = o.row_hash(o.row_words(X.astype(np.float32), "f32"))
    seed, head, tensor = 77, 3, o.TENSOR_K
    opts = o.ClusterOpts(power_iters=0, seed=seed)
    tr = o.TreeTrace()
    o.cluster_tree(X, np.eye(d), hashes, c, opts, head, tensor, tr)
    want = {}
    for level, nodes in enumerate(o.tree_levels(N, c)):
        for nd in nodes:
            if nd.n <= c:
                continue
            rv = o.warm_vector(seed, head, tensor, level, nd.index, d)
            rh = rv / np.linalg.norm(rv)
            u = tr.dirs[(level, nd.index)]
            assert math.isclose(np.linalg.norm(u), 1.0, rel_tol=1e-12)
            if level == 0:
                assert np.allclose(u, rh, rtol=0, atol=1e-14), "root starts at r/|r|"
            else:
                par = want[(level - 1, nd.index // 2)]
                assert math.isclose(u @ par, u @ rh, rel_tol=1e-10) and u @ rh > 0, "bisector"
                B = np.stack([par, rh], axis=1)
                res = u - B @ np.linalg.lstsq(B, u, rcond=None)[0]
                assert np.linalg.norm(res) < 1e-12, "in span(parent, r)"
            want[(level, nd.index)] = u
    assert len(want) == sum(nd.n > c for lv in o.tree_levels(N, c) for nd in lv)
    # p = 8 power iterations on a node whose centred covariance is isotropic
    # (M = I, whole node sampled): the start is already a fixed point
    Xi = np.concatenate([np.eye(d), -np.eye(d)]) * 2.0 + 0.75
    hi = o.row_hash(o.row_words(Xi.astype(np.float32), "f32"))
    tr8 = o.TreeTrace()
    o.cluster_tree(Xi, np.eye(d), hi, d, o.ClusterOpts(power_iters=8, seed=seed, sample_factor=2),
                   head, tensor, tr8)
    rv = o.warm_vector(seed, head, tensor, 0, 0, d)
    assert np.allclose(tr8.dirs[(0, 0)], rv / np.linalg.norm(rv), rtol=0, atol=1e-12)


def test_warm_start_composition():
    check_warm_start_composition()


def test_key_share_traces():
    # every head's query tree is traced; the heads of a group share the key tree
    r = _rng(43)
    B, H, N, D, c = 1, 4, 96, 8, 16
    Q = r.standard_normal((B, H, N, D)).astype(np.float32)
    K = np.repeat(r.standard_normal((B, 1, N, D)).astype(np.float32), H, axis=1)
    traces = {}
    pq, pk = o.cluster(Q, K, c, o.ClusterOpts(seed=5), "f32", traces=traces, key_share=2)
    for h in range(H):
        assert np.array_equal(traces[(0, h, o.TENSOR_Q)].perms[-1], pq[0, h])
        assert np.array_equal(traces[(0, h, o.TENSOR_K)].perms[-1], pk[0, h])
        assert traces[(0, h, o.TENSOR_K)] is traces[(0, h - h % 2, o.TENSOR_K)]
    assert not np.array_equal(pk[0, 0], pk[0, 2])


def test_power_iteration_zero_covariance_keeps_warm_start():
    u0 = np.ones(4) / 2.0
    X = np.tile(np.arange(4.0), (10, 1))
    assert np.array_equal(o.principal_direction(X, np.eye(4), u0, 8), u0)


# ---------------------------------------------------------------------------
# Diagonalized splitting (v1 §3.2.1 "Diagonalized recursive splitting";
# rev §4.1.1): principal-component basis and highest-variance coordinate
# ---------------------------------------------------------------------------

def _orthonormal(r, n, d):
    q, _ = np.linalg.qr(r.standard_normal((n, d)))
    return q


def check_pc_basis_known_axes():
    # X built with covariance exactly U diag(sig^2) U^T: in the identity
    # geometry the basis is U itself, columns by decreasing sig, signed so
    # that the largest-magnitude entry is positive
    r = _rng(40)
    N, d = 300, 6
    U = _orthonormal(r, d, d)
    sig = np.array([5.0, 3.5, 2.0, 1.2, 0.7, 0.3])
    H = r.standard_normal((N, d))
    Hc, _ = np.linalg.qr(H - H.mean(0))
    Hc = Hc - Hc.mean(0)   # centred columns, orthonormal up to rounding
    X = math.sqrt(N) * (Hc * sig) @ U.T + r.standard_normal(d)
    A, lam = o.pc_basis(X, np.eye(d))
    assert np.allclose(lam, sig ** 2, rtol=1e-9)
    for j in range(d):
        u = U[:, j] * (1.0 if U[np.argmax(np.abs(U[:, j])), j] > 0 else -1.0)
        assert np.allclose(A[:, j], u, atol=1e-9)


def check_pc_basis_decorrelates():
    # In a metric geometry (rank-deficient too) the coordinates y = x A are
    # uncorrelated with variances lam in decreasing order, and A = R W with
    # W orthonormal (A^T M^+ A = I on the range of M); each a_j has its
    # largest-magnitude entry positive
    r = _rng(41)
    N, d = 400, 7
    X = r.standard_normal((N, d)) @ r.standard_normal((d, d)) + r.standard_normal(d)
    for rank in (d, d - 2):
        B = r.standard_normal((d, rank))
        M = B @ B.T / rank
        A, lam = o.pc_basis(X, M)
        Y = X @ A
        Yc = Y - Y.mean(0)
        C = Yc.T @ Yc / N
        assert np.allclose(C, np.diag(lam), atol=1e-9 * lam.max())
        assert np.all(np.diff(lam) <= 1e-12 * lam.max())
        R = o.root_matrix(M)
        W = np.linalg.pinv(R) @ A
        keep = lam > 1e-9 * lam.max()
        Wk = W[:, keep]
        assert np.allclose(Wk.T @ Wk, np.eye(keep.sum()), atol=1e-8)
        for j in np.flatnonzero(keep):
            k = np.argmax(np.abs(A[:, j]))
            assert A[k, j] > 0


def check_pc_basis_root_free():
    # The same basis from a Cholesky factor of M instead of its symmetric
    # root: with M = L L^T the vectors z = L^T x have covariance L^T C L,
    # whose eigenvectors w' give a_j = L w'_j, equal to pc_basis's columns up
    # to sign; with the sign fixed on a_j they agree exactly
    r = _rng(43)
    N, d = 500, 6
    X = r.standard_normal((N, d)) @ r.standard_normal((d, d)) + r.standard_normal(d)
    B = r.standard_normal((d, d))
    M = B @ B.T / d + 0.1 * np.eye(d)
    A, lam = o.pc_basis(X, M)
    L = np.linalg.cholesky(M)
    Z = X @ L
    Zc = Z - Z.mean(0)
    lw, Wp = np.linalg.eigh(Zc.T @ Zc / N)
    idx = np.argsort(-lw)
    A2 = L @ Wp[:, idx]
    for j in range(d):
        k = np.argmax(np.abs(A2[:, j]))
        if A2[k, j] < 0:
            A2[:, j] = -A2[:, j]
    assert np.allclose(lam, lw[idx], rtol=1e-9)
    assert np.allclose(A, A2, atol=1e-9 * np.abs(A).max())


def check_diag_direction_bruteforce():
    r = _rng(42)
    for trial in range(50):
        m, d = int(r.integers(2, 9)), int(r.integers(2, 6))
        Xs = r.standard_normal((m, d))
        A = r.standard_normal((d, d))
        if trial % 5 == 0:
            A[:, 2 % d] = A[:, 0]       # an exact tie: the lower index wins
        var = []
        for j in range(d):
            y = [sum(Xs[i, k] * A[k, j] for k in range(d)) for i in range(m)]
            mu = sum(y) / m
            var.append(sum((v - mu) ** 2 for v in y) / m)
        best = max(var)
        want = min(j for j in range(d) if var[j] >= best - 1e-12 * max(1.0, best))
        j, u = o.diag_direction(Xs, A)
        assert j == want and np.array_equal(u, A[:, j])


def test_pc_basis_known_axes():
    check_pc_basis_known_axes()


def test_pc_basis_decorrelates():
    check_pc_basis_decorrelates()


def test_pc_basis_root_free():
    check_pc_basis_root_free()


def test_diag_direction_bruteforce():
    check_diag_direction_bruteforce()


def test_diag_cluster_tree_splits():
    # Every node of the diagonalized tree splits at the (score, id) order
    # statistic of the projections onto the basis column of highest sample
    # variance, and the result is a bijection with the data-independent sizes
    r = _rng(43)
    for c in (2, 4):
        for N in (13, 32):
            X = r.standard_normal((N, 4)) @ np.diag([3.0, 2.0, 1.0, 0.5])
            hashes = o.row_hash(o.row_words(X.astype(np.float32), "f32"))
            opts = o.ClusterOpts(seed=5, split_mode="diag")
            A, _ = o.pc_basis(X, np.eye(4))
            tr = o.TreeTrace()
            perm = o.cluster_tree(X, np.eye(4), hashes, c, opts, 0, 1, tr)
            assert sorted(perm.tolist()) == list(range(N))
            for lvl, nodes in enumerate(o.tree_levels(N, c)[:len(tr.scores)]):
                before, after, sc = tr.perms[lvl], tr.perms[lvl + 1], tr.scores[lvl]
                for nd in nodes:
                    if nd.n <= c:
                        continue
                    mem = before[nd.off:nd.off + nd.n]
                    T = o.sample_members(mem, hashes, lvl, 1, 4, 1, 5)
                    j, u = o.diag_direction(X[T], A)
                    assert np.allclose(sc[nd.off:nd.off + nd.n], X[mem] @ u, rtol=0, atol=0)
                    t = o.split_size(nd.n, c)
                    order = sorted(zip((X[mem] @ u).tolist(), mem.tolist()))
                    assert after[nd.off:nd.off + t].tolist() == sorted(m for _, m in order[:t])


# ---------------------------------------------------------------------------
# Split and sampling (v1 §3.2.1; rev §4.1.1)
# ---------------------------------------------------------------------------

def check_split_by_scores_bruteforce():
    r = _rng(7)
    for trial in range(200):
        n = int(r.integers(2, 12))
        members = np.sort(r.choice(1000, n, replace=False))
        scores = r.integers(0, 4, n).astype(np.float64)     # many exact ties
        if trial % 3 == 0:
            scores = np.where(scores == 0, -0.0, scores)
        t = int(r.integers(1, n))
        left, right = o.split_by_scores(members, scores, t)
        assert len(left) == t and len(right) == n - t
        assert np.all(np.diff(left) > 0) and np.all(np.diff(right) > 0)
        sc = dict(zip(members.tolist(), (scores + 0.0).tolist()))
        for a in left:
            for b in right:
                assert (sc[a], a) < (sc[b], b)


def test_split_by_scores_bruteforce():
    check_split_by_scores_bruteforce()


def test_cluster_tree_tiny_bruteforce():
    # Every node of a tiny tree (c = 1 and 2) splits its members exactly at
    # the (score, id) order statistic, and the result is a bijection.
    r = _rng(8)
    for c in (1, 2):
        for N in (5, 9, 16):
            X = r.standard_normal((N, 3))
            hashes = o.row_hash(o.row_words(X.astype(np.float32), "f32"))
            tr = o.TreeTrace()
            perm = o.cluster_tree(X, np.eye(3), hashes, c, o.ClusterOpts(seed=3), 0, 1, tr)
            assert sorted(perm.tolist()) == list(range(N))
            for lvl, nodes in enumerate(o.tree_levels(N, c)[:len(tr.scores)]):
                before, after, sc = tr.perms[lvl], tr.perms[lvl + 1], tr.scores[lvl]
                for nd in nodes:
                    if nd.n <= c:
                        continue
                    mem = before[nd.off:nd.off + nd.n]
                    s = sc[nd.off:nd.off + nd.n]
                    t = o.split_size(nd.n, c)
                    order = sorted(zip(s.tolist(), mem.tolist()))
                    want_left = sorted(m for _, m in order[:t])
                    assert after[nd.off:nd.off + t].tolist() == want_left
                    assert sorted(after[nd.off + t:nd.off + nd.n].tolist()) == \
                        sorted(m for _, m in order[t:])


def test_sample_members_properties():
    r = _rng(9)
    N, d = 20000, 64
    W = r.integers(0, 2**32, size=(N, 8), dtype=np.uint64)
    hashes = o.row_hash(W)
    members = np.arange(N)
    counts = []
    for level in range(40):
        T = o.sample_members(members, hashes, level, 1, d, 1, 11)
        assert np.all(np.isin(T, members))
        counts.append(len(T))
    assert abs(np.mean(counts) - d) < 3 * math.sqrt(d / 40) + 1
    # independent of the order of the members
    T = o.sample_members(members, hashes, 3, 0, d, 1, 11)
    T2 = o.sample_members(members[::-1].copy(), hashes, 3, 0, d, 1, 11)
    assert np.array_equal(np.sort(T), np.sort(T2))
    # whole node when a d >= n, and duplicates are sampled all-or-none
    assert np.array_equal(o.sample_members(members[:50], hashes, 0, 0, d, 1, 11), members[:50])
    dup = np.repeat(hashes[:400], 5)
    T = o.sample_members(np.arange(2000), dup, 2, 0, d, 1, 11)
    groups = np.bincount(T // 5, minlength=400)
    assert set(groups.tolist()) <= {0, 5}


# ---------------------------------------------------------------------------
# Assignment (v1 §3.3, Eq. 18-19)
# ---------------------------------------------------------------------------

def check_centroid_scores():
    r = _rng(10)
    N, D, c = 200, 8, 32
    Q = r.standard_normal((N, D)); K = r.standard_normal((N, D))
    pq = r.permutation(N); pk = r.permutation(N)
    cq, nq = o.centroids(Q, pq, c)
    ck, nk = o.centroids(K, pk, c)
    assert nq.tolist() == [32] * 6 + [8]
    A = o.cluster_scores(cq, ck)
    for a in range(len(nq)):
        qa = Q[pq[a * c:a * c + nq[a]]]
        for j in range(len(nk)):
            kj = K[pk[j * c:j * c + nk[j]]]
            # Eq. 18: the centroid product is the mean pairwise logit
            assert math.isclose(A[a, j], np.mean(qa @ kj.T), rel_tol=1e-10, abs_tol=1e-12)
            # Eq. 19: Jensen, the mean of exp is at least exp of the mean
            tau = 1 / math.sqrt(D)
            assert np.mean(np.exp(tau * qa @ kj.T)) >= math.exp(tau * A[a, j]) * (1 - 1e-12)


def test_centroid_scores():
    check_centroid_scores()


def check_topk_bruteforce():
    r = _rng(11)
    for _ in range(300):
        n = int(r.integers(1, 12))
        k = int(r.integers(1, n + 1))
        s = r.integers(-3, 3, n).astype(np.float64)
        got = o.topk_row(s, k)
        best = max(itertools.combinations(range(n), k),
                   key=lambda sub: (sum(s[list(sub)]), tuple(-x for x in sub)))
        assert tuple(got.tolist()) == best, (s, k, got, best)


def test_topk_bruteforce():
    check_topk_bruteforce()


# Adaptive selection (v1 §3.3.2 "Selection"; later revision §4.2)

def _adaptive_inputs(r, n):
    s = r.standard_normal(n) * float(r.choice([0.3, 3.0, 30.0])) + float(r.normal(0, 5))
    if r.random() < 0.3:
        s = np.round(s, 1)                      # repeated scores
    cnt = np.full(n, 64)
    cnt[-1] = int(r.integers(1, 65))            # a short last cluster
    return s.astype(np.float32).astype(np.float64), cnt, float(r.choice([0.05, 0.125, 0.5]))


def _keys(s):
    # the 16384 score bins of the selection, in fp32 as the kernel forms them
    s32 = np.asarray(s, np.float32)
    lo, hi = s32.min(), s32.max()
    u = (s32 - lo) * (np.float32(128) / (hi - lo))
    return np.minimum(16383, np.floor(u * np.float32(128)).astype(np.int64))


def check_adaptive_direct_cutoff():
    # The two passes equal a single pass over all n_bins^2 keys: the cutoff
    # key is the lower of, per criterion, the largest key K with the total
    # over keys >= K reaching the threshold
    r = _rng(50)
    for _ in range(400):
        n = int(r.integers(1, 300))
        s, cnt, tau = _adaptive_inputs(r, n)
        recall = float(r.choice([0.0, 0.3, 0.9, 0.99, 1.0]))
        mc = int(r.integers(1, 20))
        got = o.adaptive_row(s, cnt, tau, recall, mc)
        if n <= mc or s.max() == s.min():
            assert np.array_equal(got, np.arange(n))
            continue
        key = _keys(s)
        mass = np.rint(cnt * np.exp(tau * (s - s.max())) * 2.0**40).astype(np.int64)
        cum_n = np.cumsum(np.bincount(key, minlength=16384)[::-1])[::-1]
        per_key = np.zeros(16384, np.int64)
        np.add.at(per_key, key, mass)
        cum_m = np.cumsum(per_key[::-1])[::-1]
        kc = int(np.flatnonzero(cum_n >= mc).max())
        ok = np.flatnonzero(cum_m >= int(math.floor(recall * float(mass.sum()))))
        km = int(ok.max()) if ok.size else 0
        want = np.flatnonzero(key >= min(kc, km))
        assert np.array_equal(got, want), (n, recall, mc)


def check_adaptive_guarantees():
    # count >= min_count; estimated mass >= recall x total; an upper set in
    # score; dropping the members at the cutoff key breaks a criterion;
    # monotone in the recall
    r = _rng(51)
    for _ in range(300):
        n = int(r.integers(2, 200))
        s, cnt, tau = _adaptive_inputs(r, n)
        mc = int(r.integers(1, 20))
        mass = cnt * np.exp(tau * (s - s.max()))
        prev = None
        for recall in (0.0, 0.5, 0.8, 0.95, 0.999):
            sel = o.adaptive_row(s, cnt, tau, recall, mc)
            assert len(sel) >= min(mc, n)
            assert mass[sel].sum() >= recall * mass.sum() * (1 - 1e-9)
            assert np.all(np.isin(np.flatnonzero(s > s[sel].min()), sel))
            assert np.all(np.diff(sel) > 0)
            if prev is not None:
                assert np.all(np.isin(prev, sel))
            prev = sel
            if len(sel) < n and s.max() > s.min():
                key = _keys(s)
                rest = sel[key[sel] > key[sel].min()]
                assert len(rest) < mc or mass[rest].sum() < recall * mass.sum() * (1 + 1e-9)


def check_adaptive_topk_mode():
    # recall 0 with min_count k on scores far apart (no two in one of the
    # 16384 key bins) is exact top-k; recall 1 takes every cluster
    r = _rng(52)
    for _ in range(200):
        n = int(r.integers(2, 120))
        s = r.permutation(n).astype(np.float64) * 3.0 + r.uniform(0, 0.1)
        cnt = np.full(n, 128)
        k = int(r.integers(1, n + 1))
        assert np.array_equal(o.adaptive_row(s, cnt, 0.1, 0.0, k), o.topk_row(s, k))
        assert np.array_equal(o.adaptive_row(s, cnt, 1e-3, 1.0, 1), np.arange(n))


def test_adaptive_direct_cutoff():
    check_adaptive_direct_cutoff()


def test_adaptive_guarantees():
    check_adaptive_guarantees()


def test_adaptive_topk_mode():
    check_adaptive_topk_mode()


# ---------------------------------------------------------------------------
# Attention (v1 §1.2 Eq. 1-6; App. A Eq. 21-33)
# ---------------------------------------------------------------------------

def check_dense_against_libraries():
    import torch
    Q, K, V = _random_head(12, N=96, D=16)
    O, L = o.dense_attention(Q, K, V)
    tau = 1 / 4.0
    W = _dense_weights(Q, K, tau)
    assert np.allclose(O, W @ V, rtol=1e-12, atol=1e-13)
    assert np.allclose(L, scipy.special.logsumexp(tau * Q @ K.T, axis=1), rtol=1e-13)
    t = lambda x: torch.from_numpy(x)[None, None]
    Ot = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V))[0, 0].numpy()
    assert np.allclose(O, Ot, rtol=1e-12, atol=1e-13)
    O2, _ = o.dense_attention(Q, K, V, scale=0.37)
    assert np.allclose(O2, _dense_weights(Q, K, 0.37) @ V, rtol=1e-12, atol=1e-13)


def test_dense_against_libraries():
    check_dense_against_libraries()


def _sparse_case(seed, N=256, D=16, c=32, k=3, remainder=0):
    N = N - remainder
    Q, K, V = _random_head(seed, N=N, D=D)
    r = _rng(seed + 100)
    pq = r.permutation(N); pk = r.permutation(N)
    nc = -(-N // c)
    blocks = np.stack([np.sort(r.choice(nc, k, replace=False)) for _ in range(nc)])
    return Q, K, V, pq, pk, blocks, c


def _token_set(pk, blocks_row, c, N):
    sizes = o.leaf_sizes(N, c)
    return np.concatenate([pk[j * c:j * c + sizes[j]] for j in blocks_row])


def check_sparse_error_identity():
    # Eq. 3-4: o - o_S = (1 - w_S)(o_Sbar - o_S), w from dense attention.
    for rem in (0, 13):
        Q, K, V, pq, pk, blocks, c = _sparse_case(13, remainder=rem)
        N, D = Q.shape
        tau = 1 / math.sqrt(D)
        OS, _ = o.sparse_attention(Q, K, V, pq, pk, c, blocks, compensate=False)
        W = _dense_weights(Q, K, tau)
        Od = W @ V
        qsz = o.leaf_sizes(N, c)
        for a in range(len(qsz)):
            S = _token_set(pk, blocks[a], c, N)
            Sb = np.setdiff1d(np.arange(N), S)
            for i in pq[a * c:a * c + qsz[a]]:
                wS = W[i, S].sum()
                oSb = W[i, Sb] @ V[Sb] / W[i, Sb].sum()
                assert np.allclose(Od[i] - OS[i], (1 - wS) * (oSb - OS[i]), rtol=1e-9, atol=1e-12)


def test_sparse_error_identity():
    check_sparse_error_identity()


def check_smc_error_identity():
    # Eq. 21-33 with dense-normalised weights w_i and w_c = exp(tau q.kbar_c)/Z.
    for rem in (0, 13):
        Q, K, V, pq, pk, blocks, c = _sparse_case(14, remainder=rem)
        N, D = Q.shape
        tau = 1 / math.sqrt(D)
        Oh, Lh = o.sparse_attention(Q, K, V, pq, pk, c, blocks, compensate=True)
        logits = tau * Q @ K.T
        Z = np.exp(logits).sum(1)
        W = np.exp(logits) / Z[:, None]
        Od = W @ V
        ksz = o.leaf_sizes(N, c)
        qsz = o.leaf_sizes(N, c)
        for a in range(len(qsz)):
            sel = set(blocks[a].tolist())
            S = _token_set(pk, blocks[a], c, N)
            for i in pq[a * c:a * c + qsz[a]]:
                wS = W[i, S].sum()
                rhs = np.zeros(D)
                dhat = wS
                for cl in range(len(ksz)):
                    if cl in sel:
                        continue
                    mem = pk[cl * c:cl * c + ksz[cl]]
                    kb = K[mem].mean(0); vb = V[mem].mean(0)
                    wc = math.exp(tau * Q[i] @ kb) / Z[i]
                    wbar = W[i, mem].mean()
                    delta = wbar - wc
                    assert delta >= -1e-15          # Eq. 19/25: Jensen
                    cov = ((W[i, mem] - wbar)[:, None] * (V[mem] - vb)).mean(0)
                    rhs += len(mem) * (delta * (vb - Od[i]) + cov)
                    dhat += len(mem) * wc
                assert dhat <= 1 + 1e-12             # Eq. 28: d_hat <= 1
                assert np.allclose(Od[i] - Oh[i], rhs / dhat, rtol=1e-8, atol=1e-12)   # Eq. 33
                # LSE of the compensated softmax is log(Z d_hat) + the row's log scale
                assert math.isclose(Lh[i], math.log(Z[i] * dhat), rel_tol=1e-12)


def test_smc_error_identity():
    check_smc_error_identity()


def check_special_cases_equal_dense():
    Q, K, V, pq, pk, blocks, c = _sparse_case(15, N=200, c=32)
    N = Q.shape[0]
    Od, Ld = o.dense_attention(Q, K, V)
    nc = -(-N // c)
    allb = np.tile(np.arange(nc), (nc, 1))
    for comp in (False, True):
        O, L = o.sparse_attention(Q, K, V, pq, pk, c, allb, comp)
        assert np.allclose(O, Od, rtol=1e-12, atol=1e-12) and np.allclose(L, Ld, rtol=1e-12)
    # c = 1 with compensation equals dense for any k (each centroid is a token)
    N = 24
    Q, K, V = Q[:N], K[:N], V[:N]
    Od, _ = o.dense_attention(Q, K, V)
    for k in (1, 5, 24):
        Os, _, _, _, _ = o.forward(Q[None, None], K[None, None], V[None, None], 1, k, True,
                                   o.ClusterOpts(seed=2), dtype="f32")
        assert np.allclose(Os[0, 0], Od, rtol=1e-10, atol=1e-12)


def test_special_cases_equal_dense():
    check_special_cases_equal_dense()


def check_unequal_cluster_sizes():
    # Query clusters of c and key clusters of c_k != c: selecting every key
    # cluster equals dense; key clusters of one token (c_k = 1) with
    # compensation equal dense for any selection; one selected key cluster
    # per query cluster against the logits built by hand from the members
    r = _rng(17)
    N, D = 200, 16
    Q, K, V = (r.standard_normal((N, D)) for _ in range(3))
    Od, Ld = o.dense_attention(Q, K, V)
    pq = r.permutation(N)
    for c, ck in ((32, 64), (16, 64), (64, 32)):
        pk = r.permutation(N)
        nq, nk = -(-N // c), -(-N // ck)
        allb = np.tile(np.arange(nk), (nq, 1))
        for comp in (False, True):
            O, L = o.sparse_attention(Q, K, V, pq, pk, c, allb, comp, c_k=ck)
            assert np.allclose(O, Od, rtol=1e-12, atol=1e-12) and np.allclose(L, Ld, rtol=1e-12)
        one = r.integers(0, nk, size=(nq, 1))
        O, _ = o.sparse_attention(Q, K, V, pq, pk, c, one, False, c_k=ck)
        for a in range(nq):
            qi = pq[a * c:(a + 1) * c]
            j = int(one[a, 0])
            ki = pk[j * ck:(j + 1) * ck]
            want, _ = o._softmax_combine(Q[qi] @ K[ki].T / math.sqrt(D), V[ki])
            assert np.allclose(O[qi], want, rtol=1e-12, atol=1e-12)
    pk = r.permutation(N)
    for k in (1, 7, 50):
        sel = np.stack([np.sort(r.choice(N, k, replace=False)) for _ in range(-(-N // 32))])
        O, _ = o.sparse_attention(Q, K, V, pq, pk, 32, sel, True, c_k=1)
        assert np.allclose(O, Od, rtol=1e-10, atol=1e-12)


def test_unequal_cluster_sizes():
    check_unequal_cluster_sizes()


def check_piecewise_constant_keys():
    # Keys with n_c distinct rows, each repeated c times (shuffled): every split
    # keeps the copies together, so each cluster is one distinct key, delta_c = 0
    # and Cov_c = 0 (Eq. 27) and compensated attention equals dense for any k.
    r = _rng(16)
    c, nc, D = 8, 12, 16
    N = c * nc
    base = r.standard_normal((nc, D)).astype(np.float32)
    K = np.repeat(base, c, axis=0)
    sh = r.permutation(N)
    K = K[sh].astype(np.float64)
    Q = r.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    V = r.standard_normal((N, D))
    Od, _ = o.dense_attention(Q, K, V)
    for k in (1, 3, 7):
        Os, _, pq, pk, _ = o.forward(Q[None, None], K[None, None], V[None, None], c, k, True,
                                     o.ClusterOpts(seed=4), dtype="f32")
        for j in range(nc):
            assert len({tuple(x) for x in K[pk[0, 0, j * c:(j + 1) * c]]}) == 1
        assert np.allclose(Os[0, 0], Od, rtol=1e-10, atol=1e-12)


def test_piecewise_constant_keys():
    check_piecewise_constant_keys()


def check_permutation_equivariance():
    r = _rng(17)
    N, D, c = 256, 16, 32
    Q = r.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    K = r.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    V = r.standard_normal((N, D))
    P = r.permutation(N)
    args = dict(c=c, topk=3, compensate=True, opts=o.ClusterOpts(seed=9), dtype="f32")
    O1, L1, *_ = o.forward(Q[None, None], K[None, None], V[None, None], **args)
    O2, L2, *_ = o.forward(Q[P][None, None], K[P][None, None], V[P][None, None], **args)
    assert np.allclose(O2[0, 0], O1[0, 0][P], rtol=1e-12, atol=1e-12)
    assert np.allclose(L2[0, 0], L1[0, 0][P], rtol=1e-12)


def test_permutation_equivariance():
    check_permutation_equivariance()


def test_power_of_two_scaling_invariance():
    # Full-sample mode (a d >= N): scaling Q by 2^alpha and K by 2^beta scales
    # every intermediate exactly, so perms and blocks are identical.
    r = _rng(18)
    N, D, c = 64, 16, 4
    Q = r.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    K = r.standard_normal((N, D)).astype(np.float32).astype(np.float64)
    V = r.standard_normal((N, D))
    opts = o.ClusterOpts(seed=1, sample_factor=4)
    _, _, pq, pk, bl = o.forward(Q[None, None], K[None, None], V[None, None], c, 3, True, opts, "f32")
    _, _, pq2, pk2, bl2 = o.forward(8 * Q[None, None], 0.25 * K[None, None], V[None, None], c, 3,
                                    True, opts, "f32")
    assert np.array_equal(pq, pq2) and np.array_equal(pk, pk2) and np.array_equal(bl, bl2)


def test_random_cluster_control_all_selected_is_dense():
    import synth
    Q, K, V = _random_head(19, N=192, D=16)
    pq = synth.random_perm(1, 1, 1, 192)[0, 0]
    pk = synth.random_perm(2, 1, 1, 192)[0, 0]
    nc = 192 // 32
    O, _ = o.sparse_attention(Q, K, V, pq, pk, 32, np.tile(np.arange(nc), (nc, 1)), True)
    assert np.allclose(O, o.dense_attention(Q, K, V)[0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle must fail some pin.
# ---------------------------------------------------------------------------

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def _no_log_count(Q, K, V, perm_q, perm_k, c, blocks, compensate, scale=None):
    # compensation without the ln|c| cluster-size weight
    real_log = np.log
    try:
        o.np.log = lambda x: np.zeros_like(np.asarray(x, np.float64))
        return _orig["sparse_attention"](Q, K, V, perm_q, perm_k, c, blocks, compensate, scale)
    finally:
        o.np.log = real_log


_orig = {name: getattr(o, name) for name in
         ["sparse_attention", "split_size", "metric_matrices", "principal_direction", "topk_row",
          "centroids", "dense_attention", "split_by_scores", "fmix64", "pc_basis",
          "diag_direction", "adaptive_row", "cluster_masses", "head_representations",
          "warm_start"]}


def _basis_ascending(X, M):
    A, lam = _orig["pc_basis"](X, M)
    return A[:, ::-1].copy(), lam[::-1].copy()


def _basis_sign_on_w(X, M):
    # the former reading: each eigenvector w_j signed, not a_j = R w_j
    X = np.asarray(X, np.float64)
    R = o.root_matrix(M)
    Z = X @ R
    Zc = Z - Z.mean(0)
    lam, W = np.linalg.eigh(Zc.T @ Zc / X.shape[0])
    order = np.argsort(-lam, kind="stable")
    lam, W = lam[order], W[:, order]
    for j in range(W.shape[1]):
        k = int(np.argmax(np.abs(W[:, j])))
        if W[k, j] < 0:
            W[:, j] = -W[:, j]
    return R @ W, lam


def _basis_without_root(X, M):
    return _orig["pc_basis"](X, np.eye(M.shape[0]))


def _adaptive_higher_cutoff(scores, counts, tau, recall, min_count, nbins=128):
    # the upper of the two criteria's cutoffs: one criterion left unmet
    a = _orig["adaptive_row"](scores, counts, tau, recall, 1, nbins)
    b = _orig["adaptive_row"](scores, counts, tau, 0.0, min_count, nbins)
    return a if len(a) < len(b) else b


def _masses_without_counts(scores, counts, tau):
    s = np.asarray(scores, np.float64)
    return np.exp(tau * (s - s.max()))


def _direction_lowest_variance(Xs, A):
    Y = np.asarray(Xs, np.float64) @ A
    var = ((Y - Y.mean(axis=0)) ** 2).mean(axis=0)
    j = int(np.argmin(var))
    return j, A[:, j].copy()


def _direction_uncentred(Xs, A):
    Y = np.asarray(Xs, np.float64) @ A
    j = int(np.argmax((Y ** 2).mean(axis=0)))
    return j, A[:, j].copy()


def _split_size_larger(n, c):
    t = _orig["split_size"](n, c)
    if (n // c) % 2 == 1 and n % c == 0:
        t += c
    return t


def _metric_uncentred(Q, K):
    Mq, _, kbar = _orig["metric_matrices"](Q, K)
    K = np.asarray(K, np.float64)
    return Mq, K.T @ K / K.shape[0], kbar


def _power_without_metric(Xs, M, u0, p):
    return _orig["principal_direction"](Xs, np.eye(M.shape[0]), u0, p)


def _topk_ties_high(scores, k):
    s = np.asarray(scores, np.float64)
    idx = np.arange(s.shape[0])
    return np.sort(np.lexsort((-idx, -s))[:k])


def _centroids_divide_by_c(X, perm, c):
    cent, cnt = _orig["centroids"](X, perm, c)
    return cent * cnt[:, None] / c, cnt


def _dense_no_scale(Q, K, V, scale=None):
    return _orig["dense_attention"](Q, K, V, scale=1.0)


def _split_reversed(members, scores, t):
    return _orig["split_by_scores"](members, -np.asarray(scores), t)


def _fmix_wrong_shift(z):
    if isinstance(z, (int, np.integer)) and not isinstance(z, np.ndarray):
        z = int(z) & o.MASK64
        z = ((z ^ (z >> 31)) * o.MIX1) & o.MASK64
        z = ((z ^ (z >> 27)) * o.MIX2) & o.MASK64
        return z ^ (z >> 31)
    return _orig["fmix64"](z)


def _repr_no_normaliser(Q, K, opts):
    # queries split as raw q (the Eq. 16 normaliser dropped)
    Xq, Gq, Xk, Gk = _orig["head_representations"](Q, K, opts)
    return np.asarray(Q, np.float64), Gq, Xk, Gk


def _repr_uncentred_query_geometry(Q, K, opts):
    # queries under K^T K / N instead of the centred K_c^T K_c / N
    Xq, Gq, Xk, Gk = _orig["head_representations"](Q, K, opts)
    K = np.asarray(K, np.float64)
    G = K.T @ K / K.shape[0] if opts.transform else Gq
    s = o.query_normalisers(Q, G) if opts.query_normalize else np.ones(len(Q))
    return s[:, None] * np.asarray(Q, np.float64), G, Xk, Gk


def _repr_swapped_geometries(Q, K, opts):
    Xq, Gq, Xk, Gk = _orig["head_representations"](Q, K, opts)
    s = o.query_normalisers(Q, Gk) if opts.query_normalize else np.ones(len(Q))
    return s[:, None] * np.asarray(Q, np.float64), Gk, Xk, Gq


def _warm_start_no_parent(seed, head, tensor, level, index, d, parent):
    return _orig["warm_start"](seed, head, tensor, level, index, d, None)


def _warm_start_unnormalised(seed, head, tensor, level, index, d, parent):
    u = _orig["warm_start"](seed, head, tensor, level, index, d, None)
    return u if parent is None else parent + u


def _warm_start_parent_only(seed, head, tensor, level, index, d, parent):
    u = _orig["warm_start"](seed, head, tensor, level, index, d, None)
    return u if parent is None else parent.copy()


PLANTED = [
    ("sparse_attention", _no_log_count, check_smc_error_identity),
    ("split_size", _split_size_larger, check_tree_layout),
    ("metric_matrices", _metric_uncentred, check_metrics),
    ("principal_direction", _power_without_metric, check_power_iteration_matches_eigh),
    ("topk_row", _topk_ties_high, check_topk_bruteforce),
    ("centroids", _centroids_divide_by_c, check_smc_error_identity),
    ("dense_attention", _dense_no_scale, check_dense_against_libraries),
    ("split_by_scores", _split_reversed, check_split_by_scores_bruteforce),
    ("fmix64", _fmix_wrong_shift, check_splitmix64_published),
    ("pc_basis", _basis_ascending, check_pc_basis_known_axes),
    ("pc_basis", _basis_without_root, check_pc_basis_decorrelates),
    ("pc_basis", _basis_sign_on_w, check_pc_basis_decorrelates),
    ("diag_direction", _direction_lowest_variance, check_diag_direction_bruteforce),
    ("diag_direction", _direction_uncentred, check_diag_direction_bruteforce),
    ("adaptive_row", _adaptive_higher_cutoff, check_adaptive_guarantees),
    ("cluster_masses", _masses_without_counts, check_adaptive_direct_cutoff),
    ("head_representations", _repr_no_normaliser, check_head_representations),
    ("head_representations", _repr_uncentred_query_geometry, check_head_representations),
    ("head_representations", _repr_swapped_geometries, check_head_representations),
    ("head_representations", _repr_no_normaliser, check_cluster_matches_textbook_pddp),
    ("head_representations", _repr_uncentred_query_geometry, check_cluster_matches_textbook_pddp),
    ("head_representations", _repr_swapped_geometries, check_cluster_matches_textbook_pddp),
    ("warm_start", _warm_start_no_parent, check_warm_start_composition),
    ("warm_start", _warm_start_unnormalised, check_warm_start_composition),
    ("warm_start", _warm_start_parent_only, check_warm_start_composition),
]


@pytest.mark.parametrize("name,mutant,check", PLANTED,
                         ids=[f"{p[0]}-{p[1].__name__.lstrip('_')}" for p in PLANTED])
def test_planted_mistakes(monkeypatch, name, mutant, check):
    check()                                   # the pin passes on the real oracle
    monkeypatch.setattr(o, name, mutant)
    assert _fails(check), f"planted mistake in {name} was not caught"
