"""GPU parity at the full sizes of the workloads, in the launch configuration
bench.py times (one ca_cluster, ca_route, ca_attend over every head).

The oracle cannot redo a whole workload in seconds, so the outputs are
checked on samples it can compute one by one, plus properties that hold at
any size (paper: "ClusterAttention: A training-free speedup of bidirectional
attention", arXiv 2608.26965 v1):

* every split of every level of the sampled heads is bit-exact when the
  oracle's select-and-partition is fed the GPU's fp32 projections, and the
  oracle's fp64 direction for a sample of nodes, given the GPU's membership
  and parent estimate, reproduces the GPU's direction;
* routing of every head is bit-exact given the GPU's score matrix;
* attention of sampled query clusters matches the oracle on the GPU's
  clusters to max-abs 2e-2 (bf16), the LSE to 1e-2;
* permutations are bijections, clusters keep ascending token order, blocks
  are ascending, distinct and in range, for every head.
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle.clusterattn as o
import synth

pytestmark = pytest.mark.gpu

# workload, sampled heads, direction replays per level, sampled query clusters
FULL = {
    "video_32760": ((0, 21), 12, 24),
    "tabular_64k": ((5,), 12, 24),
    "tabular_256k": ((3,), 8, 12),
}


def _log(msg):
    print(msg, flush=True)


def _generate(w):
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        parts = list(ex.map(lambda h: synth.generate(w, heads=slice(h, h + 1)), range(w.H)))
    return tuple(np.concatenate([p[i] for p in parts], axis=1) for i in range(3))


def _np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


@pytest.mark.parametrize("wname", list(FULL))
def test_full_size_sampled(ca, wname):
    import torch
    heads, ndir, nclus = FULL[wname]
    w = synth.WORKLOADS[wname]
    t0 = time.time()
    Q, K, V = _generate(w)
    _log(f"{wname}: inputs {Q.shape} in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).to(dev).contiguous() for x in (Q, K, V))
    B, H, N, D = Q.shape
    c, topk = w.c, w.topk
    res = ca.cluster(tq, tk, c, seed=w.cluster_seed, trace=True)
    blocks, scores = ca.route(res.cent_q, res.cent_k, topk, return_scores=True)
    O, lse = ca.attend(tq, tk, tv, res.perm_q, res.perm_k, c, blocks, compensate=w.compensate,
                       return_lse=True)
    torch.cuda.synchronize()
    _log(f"{wname}: GPU path done")
    L = ca.tree_levels(N, c)
    S = 1 << max(L - 1, 0)
    tp = _np(res.trace_perm).reshape(L + 1, 2 * B * H, N)
    ts = _np(res.trace_score).reshape(L, 2 * B * H, N)
    td = _np(res.trace_dir).reshape(L, 2 * B * H, S, D)
    pq, pk, bl, sc = _np(res.perm_q), _np(res.perm_k), _np(blocks), _np(scores)
    Og, Lg = _np(O), _np(lse)
    nc = -(-N // c)
    sizes = o.leaf_sizes(N, c)

    # properties of every head
    for b in range(B):
        for h in range(H):
            for perm in (pq[b, h], pk[b, h]):
                assert np.array_equal(np.sort(perm), np.arange(N))
                for j, nj in enumerate(sizes):
                    assert np.all(np.diff(perm[j * c:j * c + nj]) > 0)
            assert np.all(np.diff(bl[b, h], axis=1) > 0)
            assert bl[b, h].min() >= 0 and bl[b, h].max() < nc
            # routing: bit-exact top-k given the GPU's scores
            assert np.array_equal(bl[b, h], o.route(None, None, topk, scores=sc[b, h]))
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(Lg))
    _log(f"{wname}: properties and routing of {B * H} heads ok")

    opts = o.ClusterOpts(seed=w.cluster_seed)
    levels = o.tree_levels(N, c)
    rng = np.random.default_rng(11)
    for h in heads:
        head = h   # B = 1
        Xq, Gq, Xk, Gk = o.head_representations(Q[0, h], K[0, h], opts)
        hq = o.row_hash(o.row_words(Q[0, h], w.dtype))
        hk = o.row_hash(o.row_words(K[0, h], w.dtype))
        for tensor, X, G, hs in ((0, Xq, Gq, hq), (1, Xk, Gk, hk)):
            tree = 2 * head + tensor
            for lvl in range(L):
                before, after, scl = tp[lvl, tree], tp[lvl + 1, tree], ts[lvl, tree]
                splitting = [nd for nd in levels[lvl] if nd.n > c]
                replay = set(rng.choice(len(splitting), size=min(ndir, len(splitting)),
                                        replace=False).tolist())
                for k, nd in enumerate(splitting):
                    sl = slice(nd.off, nd.off + nd.n)
                    mem = before[sl].astype(np.int64)
                    t = o.split_size(nd.n, c)
                    left, right = o.split_by_scores(mem, scl[sl].astype(np.float64), t)
                    assert np.array_equal(after[nd.off:nd.off + t], left), (wname, h, lvl, tensor)
                    assert np.array_equal(after[nd.off + t:nd.off + nd.n], right)
                    if k in replay:
                        par = td[lvl - 1, tree, nd.index // 2].astype(np.float64) if lvl else None
                        T = o.sample_members(mem, hs, lvl, tensor, D, opts.sample_factor, opts.seed)
                        u0 = o.warm_start(opts.seed, head, tensor, lvl, nd.index, D, par)
                        u = o.principal_direction(X[T], G, u0, opts.power_iters)
                        ug = td[lvl, tree, nd.index].astype(np.float64)
                        assert 1 - abs(u @ ug) / np.linalg.norm(ug) <= 1e-9, (wname, h, lvl, tensor)
                        so = X[mem] @ u
                        assert np.max(np.abs(so - scl[sl])) <= 1e-4 * (np.std(so) + 1e-30)
        _log(f"{wname}: head {h}: every split of {L} levels bit-exact, directions ok")
        # attention of sampled query clusters on the GPU's clusters
        cl = np.sort(rng.choice(nc, size=min(nclus, nc), replace=False))
        Oo, Lo = o.sparse_attention(Q[0, h], K[0, h], V[0, h], pq[0, h], pk[0, h], c, bl[0, h],
                                    w.compensate, clusters=cl)
        rows = np.concatenate([pq[0, h][a * c:a * c + sizes[a]] for a in cl])
        err = np.max(np.abs(Og[0, h][rows] - Oo[rows]))
        lerr = np.max(np.abs(Lg[0, h][rows] - Lo[rows]))
        _log(f"{wname}: head {h}: {len(rows)} query rows max|O-oracle|={err:.2e} "
             f"max|LSE-oracle|={lerr:.2e}")
        assert err <= 2e-2 and lerr <= 1e-2
