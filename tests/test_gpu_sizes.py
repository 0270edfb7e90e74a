"""GPU parity with query clusters smaller than key clusters (the pages pair
64-token query clusters with 128-token key clusters: paper "ClusterAttention:
A training-free speedup of bidirectional attention", arXiv 2608.26965 v1
§3.1).

* Clustering: each tensor's tree follows its own cluster size and nothing
  else changes, so ca_cluster(c_q, cluster_size_k = c_k) must give, bit for
  bit, the query permutation and centroids of ca_cluster(c_q) and the key
  permutation, centroids and counts of ca_cluster(c_k) (both of which the
  equal-size parity tests check node by node against the oracle); and it
  must agree with the oracle's own fp64 trees.
* Attention: ca_attend_ex given the oracle's clusters of both sizes and the
  oracle's top-k over the n_qc x n_kc centroid scores matches the oracle to
  max-abs 2e-2 (bf16) / 1e-4 (fp32), compensation on and off.
"""
import math

import numpy as np
import pytest

import oracle.clusterattn as o
from tie_check import check_tree
import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}

CASES = {
    # name: (workload, N, heads, c_q, c_k, topk)
    "gmm_f32_d64_q64_k128": ("small_gmm_1k", 1024, 1, 64, 128, 3),
    "video_bf16_d128_q64_k128_ragged": ("video_32760", 4000, 2, 64, 128, 4),
    "gmm_bf16_d64_q64_k256_ragged": ("tabular_256k", 5000, 2, 64, 256, 3),
    "gmm_bf16_d64_q128_k256_ragged": ("tabular_64k", 3000, 2, 128, 256, 2),
}

_cache = {}


def _inputs(name):
    if name not in _cache:
        wname, N, H, cq, ck, topk = CASES[name]
        w = synth.WORKLOADS[wname]
        Q, K, V = synth.generate(w, heads=slice(0, H), N=N)
        _cache[name] = (w, Q, K, V, cq, ck, topk)
    return _cache[name]


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def _np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_sizes_match_single_size_runs(ca, name):
    import torch
    w, Q, K, V, cq, ck, topk = _inputs(name)
    tq, tk = _dev(Q, w.dtype), _dev(K, w.dtype)
    both = ca.cluster(tq, tk, cq, seed=w.cluster_seed, cluster_size_k=ck)
    qrun = ca.cluster(tq, tk, cq, seed=w.cluster_seed)
    krun = ca.cluster(tq, tk, ck, seed=w.cluster_seed)
    assert torch.equal(both.perm_q, qrun.perm_q) and torch.equal(both.cent_q, qrun.cent_q)
    assert torch.equal(both.perm_k, krun.perm_k) and torch.equal(both.cent_k, krun.cent_k)
    assert torch.equal(both.counts, krun.counts)
    B, H = Q.shape[:2]
    N = Q.shape[2]
    traces = {}
    pq, pk = o.cluster(Q, K, cq, o.ClusterOpts(seed=w.cluster_seed), w.dtype, traces=traces, c_k=ck)
    for tensor, gp, op, cc in ((o.TENSOR_Q, _np(both.perm_q), pq, cq),
                               (o.TENSOR_K, _np(both.perm_k), pk, ck)):
        for b in range(B):
            for h in range(H):
                ag, worst = check_tree(gp[b, h], op[b, h], traces[(b, h, tensor)], N, cc,
                                       (name, b, h, tensor))
                print(f"{name}: head {h} tensor {tensor}: agreement {ag:.5f}, "
                      f"largest tie distance {worst:.2e} IQR")


@pytest.mark.parametrize("compensate", [True, False])
@pytest.mark.parametrize("name", list(CASES))
def test_attend_sizes_given_oracle_clusters(ca, name, compensate):
    import torch
    w, Q, K, V, cq, ck, topk = _inputs(name)
    B, H, N, D = Q.shape
    pq, pk = o.cluster(Q, K, cq, o.ClusterOpts(seed=w.cluster_seed), w.dtype, c_k=ck)
    nq = len(o.leaf_sizes(N, cq))
    blocks = np.empty((B, H, nq, topk), np.int32)
    for b in range(B):
        for h in range(H):
            cqm, _ = o.centroids(Q[b, h], pq[b, h], cq)
            ckm, _ = o.centroids(K[b, h], pk[b, h], ck)
            blocks[b, h] = o.route(cqm, ckm, topk)
    O = ca.attend(_dev(Q, w.dtype), _dev(K, w.dtype), _dev(V, w.dtype),
                  torch.from_numpy(pq.astype(np.int32)).cuda(),
                  torch.from_numpy(pk.astype(np.int32)).cuda(), cq,
                  torch.from_numpy(blocks).cuda(), compensate=compensate, c_k=ck)
    Oo, _ = o.attend(Q, K, V, pq, pk, cq, blocks, compensate, c_k=ck)
    err = np.max(np.abs(_np(O) - Oo))
    print(f"{name} compensate={compensate}: max-abs {err:.2e}")
    assert err <= TOL[w.dtype], (name, compensate, err)


def test_query_clusters_larger_than_key_clusters_rejected(ca):
    import torch
    w, Q, K, V, cq, ck, topk = _inputs("video_bf16_d128_q64_k128_ragged")
    tq = _dev(Q, w.dtype)
    perm = torch.zeros(Q.shape[:3], dtype=torch.int32, device="cuda")
    blocks = torch.zeros((1, 2, 32, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ca.CAError):
        ca.attend(tq, tq, tq, perm, perm, 128, blocks, c_k=64)
