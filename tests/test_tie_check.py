"""The end-to-end acceptance helper on the CPU: a swap of the two tokens on
either side of a split threshold is a median tie; a swap of tokens far from
it is not."""
import numpy as np
import pytest

import oracle.clusterattn as o
from tie_check import check_tree, tie_distances


def _tree(seed=1, N=512, D=8, c=32):
    r = np.random.default_rng(seed)
    X = (r.standard_normal((N, D)) @ r.standard_normal((D, D))).astype(np.float32)
    Q, K = X[None, None], (X + 0.1)[None, None]
    traces = {}
    pq, _ = o.cluster(Q, K, c, o.ClusterOpts(seed=3), "f32", traces=traces)
    return pq[0, 0], traces[(0, 0, o.TENSOR_Q)], N, c


def _swap(perm, a, b):
    p = perm.copy()
    ia, ib = np.flatnonzero(p == a)[0], np.flatnonzero(p == b)[0]
    p[ia], p[ib] = b, a
    return p


def test_identical_trees_agree():
    perm, tr, N, c = _tree()
    assert tie_distances(perm, perm, tr, N, c) == []
    assert check_tree(perm, perm, tr, N, c) == (1.0, 0.0)


def test_threshold_swap_is_a_tie_and_far_swap_is_not():
    perm, tr, N, c = _tree()
    sc, before = tr.scores[0], tr.perms[0]
    order = np.argsort(sc, kind="stable")
    t = o.split_size(N, c)
    a, b = before[order[t - 1]], before[order[t]]       # either side of the root threshold
    d = tie_distances(_swap(perm, a, b), perm, tr, N, c)
    assert sorted(x[0] for x in d) == sorted([a, b]) and all(x[1] == 0 for x in d)
    assert max(x[2] for x in d) < 1e-2
    far_a, far_b = before[order[0]], before[order[-1]]   # the extremes of the root node
    d2 = tie_distances(_swap(perm, far_a, far_b), perm, tr, N, c)
    assert min(x[2] for x in d2) > 0.5
    with pytest.raises(AssertionError):
        check_tree(_swap(perm, far_a, far_b), perm, tr, N, c)
