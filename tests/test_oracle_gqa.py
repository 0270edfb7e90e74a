"""Pin of the oracle's shared key clustering for grouped-query attention
(paper "ClusterAttention: A training-free speedup of bidirectional
attention", arXiv 2608.26965 v1 §6.2 "Extension beyond MHA", the option of
one key clustering under the mean of the query heads' second-moment
matrices).

With the group's first head's queries all zero and the second head's
queries sqrt(D) e_j, each unit vector N/D times (so Q^T Q / N = I), the mean
metric is I / 2. The power iteration is invariant to the metric's scale
(and halving is exact), so the shared key permutation must equal the
Euclidean key clustering of the same keys with the same random draws. The
first head's metric alone is zero and no pooling at all would give the zero
or the identity metric on one head only, so either mistake changes the
result; both are planted and must be caught.
"""
import numpy as np
import pytest

import oracle.clusterattn as o


def check_shared_keys_mean_metric():
    r = np.random.default_rng(7)
    N, D, c = 512, 16, 64
    Q = np.zeros((1, 2, N, D))
    Q[0, 1] = np.sqrt(D) * np.tile(np.eye(D), (N // D, 1))
    K1 = r.standard_normal((N, D)) * (1.0 + np.arange(D)) + 0.3
    K = np.stack([K1, K1])[None]
    pq, pk = o.cluster(Q, K, c, o.ClusterOpts(seed=3), "f32", key_share=2)
    _, pk_e = o.cluster(Q[:, :1], K[:, :1], c, o.ClusterOpts(seed=3, transform=False), "f32")
    assert np.array_equal(pk[0, 0], pk_e[0, 0])
    assert np.array_equal(pk[0, 1], pk[0, 0])


def test_shared_keys_mean_metric():
    check_shared_keys_mean_metric()


def _fails():
    try:
        check_shared_keys_mean_metric()
    except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
        return True
    return False


def test_shared_keys_planted(monkeypatch):
    # the mean taken over the first head only: zero metric
    real_cluster = o.cluster

    def cluster_first_only(Q, K, c, opts=None, dtype="bf16", traces=None, c_k=None, key_share=1):
        if key_share > 1:
            Q = Q.copy()
            Q[:, 1::key_share] = 0.0
        return real_cluster(Q, K, c, opts, dtype, traces, c_k, key_share)

    monkeypatch.setattr(o, "cluster", cluster_first_only)
    assert _fails()
