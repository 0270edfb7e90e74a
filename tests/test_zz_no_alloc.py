"""ca_route_noalloc (the routing call for callers that cannot allocate)
against ca_route through the C ABI: the selected blocks are bit-identical on
two calls in a row, the second with a smaller input, and a call beyond the
scratch maximum is refused before anything runs."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _cents(torch, seed, B, H, nq, nk, D):
    g = torch.Generator().manual_seed(seed)
    cq = torch.randn((B, H, nq, D), generator=g, dtype=torch.float32)
    ck = torch.randn((B, H, nk, D), generator=g, dtype=torch.float32)
    # a few exact ties in each row: equal key centroids
    if nk > 1:
        ck[:, :, 1] = ck[:, :, 0]
    return cq.cuda(), ck.cuda()


@pytest.mark.parametrize("first,second", [
    ((1, 40, 256, 256, 128, 32), (1, 3, 64, 100, 64, 7)),      # headline routing shape, then smaller
    ((2, 4, 512, 512, 64, 64), (1, 1, 1, 1, 64, 1)),
])
def test_route_noalloc_matches_route(ca, first, second):
    import torch
    for k, (B, H, nq, nk, D, topk) in enumerate((first, second)):
        print(f"route_noalloc call {k}: B={B} H={H} n_qc={nq} n_kc={nk} D={D} topk={topk}", flush=True)
        cq, ck = _cents(torch, 100 + k, B, H, nq, nk, D)
        want = ca.route(cq, ck, topk)
        out = torch.full((B, H, nq, topk), -7, dtype=torch.int32, device="cuda")
        got = ca.route_noalloc(cq, ck, topk, blocks=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(got, want)
        b = got.cpu().numpy()
        assert np.all(np.diff(b, axis=-1) > 0) and b.min() >= 0 and b.max() < nk


def test_route_noalloc_rejects_beyond_scratch(ca):
    import torch
    cq = torch.zeros((1, 9, 1024, 64), device="cuda")
    ck = torch.zeros((1, 9, 1024, 64), device="cuda")
    out = torch.full((1, 9, 1024, 4), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(ca.CAError, match="scratch"):
        ca.route_noalloc(cq, ck, 4, blocks=out)
    torch.cuda.synchronize()
    assert int(out.min()) == -7 and int(out.max()) == -7     # nothing ran
