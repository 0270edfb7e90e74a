"""GPU routing on centroid matrices of every row length the library takes.

The top-k of a query cluster (v1 §3.3.2: the k key clusters of largest mean
logit q̄·k̄, Eq. 18; ties to the lower index, written ascending) runs on one
wave per row for rows of at most 1024 key clusters and on one workgroup per
row above that. Both are checked against the oracle's top-k fed the GPU's
own score matrix, bit for bit, on centroids drawn on a coarse grid so that
equal scores (and so the tie rule) occur in every row.
"""
import numpy as np
import pytest

import oracle.clusterattn as o

pytestmark = pytest.mark.gpu


def _centroids(n, d, seed):
    rng = np.random.default_rng(seed)
    # small integers: exact products and sums in fp32, many equal scores
    return rng.integers(-2, 3, size=(1, 2, n, d)).astype(np.float32)


@pytest.mark.parametrize("n_kc", [1000, 1024, 1025, 3000])
@pytest.mark.parametrize("topk", [1, 37, "all"])
def test_route_matches_oracle_topk(ca, n_kc, topk):
    import torch
    k = n_kc if topk == "all" else topk
    cq = torch.from_numpy(_centroids(6, 64, 7)).cuda()
    ck = torch.from_numpy(_centroids(n_kc, 64, 11 + n_kc)).cuda()
    blocks, scores = ca.route(cq, ck, k, return_scores=True)
    bl = blocks.cpu().numpy()
    sc = scores.cpu().numpy()
    assert np.array_equal(sc, np.einsum("bhqd,bhkd->bhqk", cq.cpu().numpy().astype(np.float64),
                                        ck.cpu().numpy().astype(np.float64)))
    ties = 0
    for h in range(2):
        want = o.route(None, None, k, scores=sc[0, h])
        assert np.array_equal(bl[0, h], want), (h, n_kc, k)
        ties += sum(len(r) - len(np.unique(r)) for r in sc[0, h])
    assert ties > 0   # the rows do hold equal scores


def test_route_workspace_path_matches_scores_path(ca):
    """The workspace call (scores in scratch) selects the same clusters."""
    import torch
    cq = torch.from_numpy(_centroids(9, 128, 3)).cuda()
    ck = torch.from_numpy(_centroids(1300, 128, 5)).cuda()
    a = ca.route(cq, ck, 50)
    b, _ = ca.route(cq, ck, 50, return_scores=True)
    assert torch.equal(a, b)
