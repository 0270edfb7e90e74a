"""The forward (ca_cluster -> ca_route or ca_route_adaptive -> ca_attend) captured
in a HIP graph for fixed shapes and replayed: every call enqueues kernels
only (no host synchronisation, no allocation, no memset inside the library),
so the captured forward must reproduce the eager one bit for bit on every
replay, with the program's own eager work and synchronisations between the
replays."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _forward(ca, Q, K, V, c, topk, split_mode, assign):
    cr = ca.cluster(Q, K, c, seed=7, split_mode=split_mode, query_normalize=assign == "topk")
    if assign == "topk":
        blocks, nsel = ca.route(cr.cent_q, cr.cent_k, topk), None
    else:
        blocks, nsel = ca.route_adaptive(cr.cent_q, cr.cent_k, cr.counts, 0.9, min_count=4)
    O = ca.attend(Q, K, V, cr.perm_q, cr.perm_k, c, blocks, compensate=True, nsel=nsel)
    return O, cr.perm_q, cr.perm_k, blocks


@pytest.mark.parametrize("split_mode,assign", [("power", "topk"), ("diag", "topk"),
                                               ("power", "adaptive")])
def test_graph_replays_match_eager(ca, split_mode, assign):
    import torch
    w = synth.WORKLOADS["video_32760"]
    Qn, Kn, Vn = synth.generate(w, heads=slice(0, 2), N=4000)
    dev = torch.device("cuda:0")
    Q, K, V = (torch.from_numpy(x).to(torch.bfloat16).to(dev).contiguous() for x in (Qn, Kn, Vn))
    c, topk = 128, 4
    ref = [t.clone() for t in _forward(ca, Q, K, V, c, topk, split_mode, assign)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # warm-up on the capture stream
        _forward(ca, Q, K, V, c, topk, split_mode, assign)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = _forward(ca, Q, K, V, c, topk, split_mode, assign)
    for rep in range(3):
        for t in out:                 # eager work between the replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), (split_mode, assign, rep)
        x = torch.randn(1 << 16, device=dev).sum()   # more eager work
        torch.cuda.synchronize()
    del g
