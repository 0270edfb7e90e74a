"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Inputs come from the seeded generators in ``synth`` at sizes the oracle
finishes in seconds, spanning several tiles and a ragged last cluster.
Acceptance (paper: "ClusterAttention: A training-free speedup of
bidirectional attention", arXiv 2608.26965 v1):

* splits are bit-exact when the oracle's select-and-partition is fed the GPU's
  fp32 projections; routing is bit-exact when the oracle's top-k is fed the
  GPU's score matrix;
* directions recomputed by the oracle in fp64 on the GPU's node memberships
  reproduce the GPU's split sides for >= 99.9% of tokens per level, and every
  disagreement sits at the split threshold (a median tie);
* attention given identical clusters: max-abs <= 2e-2 for bf16 inputs with
  fp32 accumulation, <= 1e-4 for the fp32 path.
"""
import math

import numpy as np
import pytest

import oracle.clusterattn as o
import synth
from tie_check import check_tree

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}

CASES = {
    # name: (workload, N, heads, c, topk)
    "gmm_f32_d64_c64": ("small_gmm_1k", 1024, 1, 64, 4),
    "gmm_bf16_d64_c128_ragged": ("tabular_64k", 3000, 2, 128, 4),
    "video_bf16_d128_c128_ragged": ("video_32760", 4000, 2, 128, 4),
    "gmm_bf16_d64_c256_ragged": ("tabular_256k", 5000, 2, 256, 3),
    "peaked_bf16_d64_c64": ("sweep_16k_peaked", 2000, 2, 64, 5),
}


def _case(name):
    wname, N, H, c, topk = CASES[name]
    w = synth.WORKLOADS[wname]
    Q, K, V = synth.generate(w, heads=slice(0, H), N=N)
    return w, Q, K, V, c, topk


_cache = {}


def _inputs(name):
    if name not in _cache:
        _cache[name] = _case(name)
    return _cache[name]


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def _np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def _opts(w):
    return o.ClusterOpts(seed=w.cluster_seed)


def _gpu_cluster(ca, name, trace=False):
    w, Q, K, V, c, topk = _inputs(name)
    return ca.cluster(_dev(Q, w.dtype), _dev(K, w.dtype), c, seed=w.cluster_seed, trace=trace)


# ---------------------------------------------------------------------------
# Clustering
# ---------------------------------------------------------------------------

def _replay_direction(X, M, hashes, members, level, tensor, head, slot, d, opts, parent):
    """The oracle's direction for one node, on a given membership."""
    T = o.sample_members(members, hashes, level, tensor, d, opts.sample_factor, opts.seed)
    u0 = o.warm_start(opts.seed, head, tensor, level, slot, d, parent)
    return o.principal_direction(X[T], M, u0, opts.power_iters)


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_against_oracle_per_level(ca, name):
    """Stage-isolated clustering parity, node by node.

    For every node the oracle is given the GPU's membership (the permutation
    before the level) and the GPU's estimate for the parent (the warm start):
    (1) its select-and-partition fed the GPU's fp32 projections reproduces the
    GPU's children bit for bit; (2) its fp64 direction reproduces the GPU's
    projections to 1e-4 of their spread; (3) splitting with its own fp64
    projections puts every token on the GPU's side except at the threshold.
    """
    w, Q, K, V, c, topk = _inputs(name)
    B, H, N, D = Q.shape
    res = _gpu_cluster(ca, name, trace=True)
    L = ca.tree_levels(N, c)
    S = 1 << max(L - 1, 0)
    # trace layouts [level][head][tensor][...] -> [level][tree = 2 head + tensor][...]
    tp = _np(res.trace_perm).reshape(L + 1, 2 * B * H, N)
    ts = _np(res.trace_score).reshape(max(L, 1), 2 * B * H, N)
    td = _np(res.trace_dir).reshape(max(L, 1), 2 * B * H, S, D)
    levels = o.tree_levels(N, c)
    opts = _opts(w)
    for b in range(B):
        for h in range(H):
            head = b * H + h
            Xq, Gq, Xk, Gk = o.head_representations(Q[b, h], K[b, h], opts)
            hq = o.row_hash(o.row_words(Q[b, h], w.dtype))
            hk = o.row_hash(o.row_words(K[b, h], w.dtype))
            for tensor, X, G, hs in ((0, Xq, Gq, hq), (1, Xk, Gk, hk)):
                tree = head * 2 + tensor
                assert np.array_equal(tp[0, tree], np.arange(N))
                disagree, total = 0, 0
                for lvl in range(L):
                    before, after, sc = tp[lvl, tree], tp[lvl + 1, tree], ts[lvl, tree]
                    moved = np.zeros(N, bool)
                    for nd in levels[lvl]:
                        if nd.n <= c:
                            continue
                        sl = slice(nd.off, nd.off + nd.n)
                        moved[sl] = True
                        mem = before[sl].astype(np.int64)
                        t = o.split_size(nd.n, c)
                        # (1) bit-exact select + partition given the GPU's scores
                        left, right = o.split_by_scores(mem, sc[sl].astype(np.float64), t)
                        assert np.array_equal(after[nd.off:nd.off + t], left), (name, lvl, tensor)
                        assert np.array_equal(after[nd.off + t:nd.off + nd.n], right)
                        # (2) oracle direction on the GPU's membership and parent estimate
                        par = td[lvl - 1, tree, nd.index // 2].astype(np.float64) if lvl else None
                        u = _replay_direction(X, G, hs, mem, lvl, tensor, head, nd.index, D, opts, par)
                        ug = td[lvl, tree, nd.index].astype(np.float64)
                        assert 1 - abs(u @ ug) / np.linalg.norm(ug) <= 1e-9, (name, lvl, tensor)
                        so = X[mem] @ u
                        sg = sc[sl].astype(np.float64)
                        spread = np.std(so) + 1e-30
                        assert np.max(np.abs(so - sg)) <= 1e-4 * spread, (name, lvl, tensor)
                        # (3) sides from the oracle's own projections
                        lo, ro = o.split_by_scores(mem, so, t)
                        bad = np.isin(mem, lo) != np.isin(mem, left)
                        disagree += int(bad.sum())
                        total += nd.n
                        if bad.any():
                            thr = np.sort(so)[t - 1:t + 1].mean()
                            iqr = np.subtract(*np.percentile(so, [75, 25])) + 1e-30
                            assert np.all(np.abs(so[bad] - thr) <= 1e-4 * iqr), (name, lvl, tensor)
                    assert np.array_equal(before[~moved], after[~moved])
                assert disagree <= 1e-3 * max(total, 1), (name, tensor, disagree, total)
                final = tp[L, tree]
                assert np.array_equal(np.sort(final), np.arange(N))
                perm = _np(res.perm_q if tensor == 0 else res.perm_k)[b, h]
                assert np.array_equal(perm, final)
                for j, nj in enumerate(o.leaf_sizes(N, c)):
                    assert np.all(np.diff(perm[j * c:j * c + nj]) > 0)


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_end_to_end_agreement(ca, name):
    """The whole GPU tree against the oracle's own fp64 tree: at least 99.9 %
    of tokens in the same cluster, and every token that differs left the
    oracle's path at a median tie (its oracle score within 1e-3 of the node's
    interquartile range from the split threshold; tests/tie_check.py). The
    node-by-node test above is the stage-isolated parity check."""
    w, Q, K, V, c, topk = _inputs(name)
    B, H, N, D = Q.shape
    res = _gpu_cluster(ca, name)
    traces = {}
    pq, pk = o.cluster(Q, K, c, _opts(w), w.dtype, traces=traces)
    for tensor, gp, op in ((o.TENSOR_Q, _np(res.perm_q), pq), (o.TENSOR_K, _np(res.perm_k), pk)):
        for b in range(B):
            for h in range(H):
                ag, worst = check_tree(gp[b, h], op[b, h], traces[(b, h, tensor)], N, c,
                                       (name, b, h, tensor))
                print(f"{name}: head {h} tensor {tensor}: agreement {ag:.5f}, "
                      f"largest tie distance {worst:.2e} IQR")


@pytest.mark.parametrize("name", list(CASES))
def test_centroids_and_route(ca, name):
    w, Q, K, V, c, topk = _inputs(name)
    B, H, N, D = Q.shape
    res = _gpu_cluster(ca, name)
    blocks, scores = ca.route(res.cent_q, res.cent_k, topk, return_scores=True)
    cq_g, ck_g = _np(res.cent_q), _np(res.cent_k)
    bl, sc = _np(blocks), _np(scores)
    cnt = _np(res.counts)
    for b in range(B):
        for h in range(H):
            cq, nq = o.centroids(Q[b, h], _np(res.perm_q)[b, h], c)
            ck, _ = o.centroids(K[b, h], _np(res.perm_k)[b, h], c)
            assert np.array_equal(cnt[b, h], nq)
            assert np.allclose(cq_g[b, h], cq, rtol=1e-5, atol=1e-5)
            assert np.allclose(ck_g[b, h], ck, rtol=1e-5, atol=1e-5)
            A = o.cluster_scores(cq_g[b, h], ck_g[b, h])
            assert np.allclose(sc[b, h], A, rtol=1e-5, atol=1e-4)
            # bit-exact top-k given the GPU's score matrix
            assert np.array_equal(bl[b, h], o.route(None, None, topk, scores=sc[b, h]))


def _tol(w):
    return TOL[w.dtype]


@pytest.mark.parametrize("compensate", [True, False])
@pytest.mark.parametrize("name", list(CASES))
def test_attend_given_oracle_clusters(ca, name, compensate):
    import torch
    w, Q, K, V, c, topk = _inputs(name)
    B, H, N, D = Q.shape
    _, _, pq, pk, blocks = o.forward(Q, K, V, c, topk, compensate, _opts(w), w.dtype)
    Og, Lg = ca.attend(_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype),
                       torch.from_numpy(pq.astype(np.int32)).cuda(),
                       torch.from_numpy(pk.astype(np.int32)).cuda(), c,
                       torch.from_numpy(blocks.astype(np.int32)).cuda(),
                       compensate=compensate, return_lse=True)
    Oo, Lo = o.attend(Q, K, V, pq, pk, c, blocks, compensate)
    err = np.max(np.abs(_np(Og) - Oo))
    lerr = np.max(np.abs(_np(Lg) - Lo))
    Od, _ = o.dense(Q, K, V)
    print(f"{name} comp={compensate}: max|O-oracle|={err:.2e} max|LSE-oracle|={lerr:.2e} "
          f"max|oracle-dense|={np.max(np.abs(Oo - Od)):.3f}")
    assert err <= _tol(w)
    assert lerr <= (1e-2 if w.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("name", list(CASES))
def test_all_selected_equals_dense(ca, name):
    import torch
    w, Q, K, V, c, topk = _inputs(name)
    B, H, N, D = Q.shape
    nc = -(-N // c)
    rng = np.random.default_rng(5)
    pq = np.stack([[rng.permutation(N) for _ in range(H)] for _ in range(B)]).astype(np.int32)
    pk = np.stack([[rng.permutation(N) for _ in range(H)] for _ in range(B)]).astype(np.int32)
    blocks = np.broadcast_to(np.arange(nc, dtype=np.int32), (B, H, nc, nc)).copy()
    Od, Ld = o.dense(Q, K, V)
    for comp in (True, False):
        Og, Lg = ca.attend(_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype),
                           torch.from_numpy(pq).cuda(), torch.from_numpy(pk).cuda(), c,
                           torch.from_numpy(blocks).cuda(), compensate=comp, return_lse=True)
        assert np.max(np.abs(_np(Og) - Od)) <= _tol(w)
        assert np.max(np.abs(_np(Lg) - Ld)) <= (1e-2 if w.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("name", list(CASES))
def test_dense_matches_oracle(ca, name):
    w, Q, K, V, c, topk = _inputs(name)
    Og, Lg = ca.dense(_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype), return_lse=True)
    Od, Ld = o.dense(Q, K, V)
    assert np.max(np.abs(_np(Og) - Od)) <= _tol(w)
    assert np.max(np.abs(_np(Lg) - Ld)) <= (1e-2 if w.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_given_gpu_clusters(ca, name):
    """Whole GPU path; the oracle attends with the GPU's perms and blocks."""
    w, Q, K, V, c, topk = _inputs(name)
    Og, cr, blocks = ca.forward(_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype), c, topk,
                                seed=w.cluster_seed, return_all=True)
    Oo, _ = o.attend(Q, K, V, _np(cr.perm_q), _np(cr.perm_k), c, _np(blocks), True)
    assert np.max(np.abs(_np(Og) - Oo)) <= _tol(w)


def test_piecewise_constant_keys_exact(ca):
    """Keys with n_c distinct rows repeated c times: every GPU key cluster is
    one group, and compensated attention equals dense for any k (Eq. 27)."""
    import torch
    rng = np.random.default_rng(7)
    c, nc, D, H = 64, 24, 64, 2
    N = c * nc
    Q = synth.bf16_round(rng.standard_normal((1, H, N, D), dtype=np.float32))
    V = synth.bf16_round(rng.standard_normal((1, H, N, D), dtype=np.float32))
    base = synth.bf16_round(rng.standard_normal((1, H, nc, D), dtype=np.float32))
    K = np.repeat(base, c, axis=2)
    for h in range(H):
        K[0, h] = K[0, h][rng.permutation(N)]
    Od, _ = o.dense(Q, K, V)
    for topk in (1, 5):
        Og, cr, blocks = ca.forward(_dev(Q, "bf16"), _dev(K, "bf16"), _dev(V, "bf16"), c, topk,
                                    seed=3, return_all=True)
        pk = _np(cr.perm_k)
        for h in range(H):
            for j in range(nc):
                rows = K[0, h][pk[0, h, j * c:(j + 1) * c]]
                assert np.all(rows == rows[0])
        assert np.max(np.abs(_np(Og) - Od)) <= 2e-2


def test_determinism(ca):
    name = "video_bf16_d128_c128_ragged"
    w, Q, K, V, c, topk = _inputs(name)
    args = (_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype), c, topk)
    O1, cr1, b1 = ca.forward(*args, seed=w.cluster_seed, return_all=True)
    O2, cr2, b2 = ca.forward(*args, seed=w.cluster_seed, return_all=True)
    import torch
    assert torch.equal(cr1.perm_q, cr2.perm_q) and torch.equal(cr1.perm_k, cr2.perm_k)
    assert torch.equal(b1, b2) and torch.equal(O1, O2)


def test_random_cluster_control(ca):
    import torch
    name = "gmm_bf16_d64_c128_ragged"
    w, Q, K, V, c, topk = _inputs(name)
    B, H, N, D = Q.shape
    pq = synth.random_perm(w.control_seed, B, H, N)
    pk = synth.random_perm(w.control_seed + 1, B, H, N)
    cqs, cks, bls = [], [], []
    blocks = np.empty((B, H, -(-N // c), topk), np.int64)
    for b in range(B):
        for h in range(H):
            cq, _ = o.centroids(Q[b, h], pq[b, h], c)
            ck, _ = o.centroids(K[b, h], pk[b, h], c)
            blocks[b, h] = o.route(cq, ck, topk)
    Og = ca.attend(_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype),
                   torch.from_numpy(pq).cuda(), torch.from_numpy(pk).cuda(), c,
                   torch.from_numpy(blocks.astype(np.int32)).cuda())
    Oo, _ = o.attend(Q, K, V, pq, pk, c, blocks, True)
    assert np.max(np.abs(_np(Og) - Oo)) <= _tol(w)
