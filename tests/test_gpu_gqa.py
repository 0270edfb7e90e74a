"""Grouped- and multi-query attention: K and V with fewer heads than Q.

The pages leave the key clustering open for shared key/value heads (paper
"ClusterAttention: A training-free speedup of bidirectional attention", arXiv
2608.26965 v1 §6.2 "Extension beyond MHA"); the option built is one key
clustering per associated query head. That is multi-head attention on K and V
repeated per query head, so:

* ca_cluster with kv_heads on the shared K must give, bit for bit, the
  permutations, centroids and counts of ca_cluster on K repeated to H heads
  (whose parity with the oracle the multi-head tests establish), for both
  split modes, bf16 and fp32;
* ca_attend_ex with kv_heads must give, bit for bit, the output and LSE of the
  attention on repeated K and V (bf16, FP8 Q.K^T, fp32; equal and unequal
  cluster sizes), and match the oracle on the repeated tensors to max-abs
  2e-2 (bf16) / 1e-4 (fp32).
"""
import numpy as np
import pytest

import oracle.clusterattn as o
from tie_check import check_tree
import synth

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, N, query heads, kv heads, dtype, c_q, c_k)
    "video_gqa4to2_bf16": ("video_32760", 3000, 4, 2, "bf16", 128, 128),
    "video_mqa4to1_bf16_q64_k128": ("video_32760", 3000, 4, 1, "bf16", 64, 128),
    "gmm_gqa4to2_f32": ("tabular_64k", 1024, 4, 2, "f32", 64, 64),
}


def _inputs(name):
    wname, N, H, Hkv, dt, cq, ck = CASES[name]
    w = synth.WORKLOADS[wname]
    Q, _, _ = synth.generate(w, heads=slice(0, H), N=N)
    # the key/value heads: the first Hkv heads' K and V of the same generator
    _, K, V = synth.generate(w, heads=slice(0, Hkv), N=N)
    return w, Q, K, V, H // Hkv, dt, cq, ck


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def _np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


@pytest.mark.parametrize("split_mode", ["power", "diag"])
@pytest.mark.parametrize("name", list(CASES))
def test_cluster_shared_heads_equal_repeated(ca, name, split_mode):
    import torch
    w, Q, K, V, G, dt, cq, ck = _inputs(name)
    tq, tk = _dev(Q, dt), _dev(K, dt)
    tk_rep = tk.repeat_interleave(G, dim=1).contiguous()
    kw = dict(seed=w.cluster_seed, split_mode=split_mode, cluster_size_k=ck if ck != cq else 0)
    shared = ca.cluster(tq, tk, cq, **kw)
    rep = ca.cluster(tq, tk_rep, cq, **kw)
    for f in ("perm_q", "perm_k", "cent_q", "cent_k", "counts"):
        assert torch.equal(getattr(shared, f), getattr(rep, f)), (name, split_mode, f)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_attend_shared_heads_equal_repeated_and_oracle(ca, name, fp8):
    import torch
    w, Q, K, V, G, dt, cq, ck = _inputs(name)
    if fp8 and dt != "bf16":
        pytest.skip("FP8 attention takes bf16 inputs")
    tq, tk, tv = _dev(Q, dt), _dev(K, dt), _dev(V, dt)
    tk_rep = tk.repeat_interleave(G, dim=1).contiguous()
    tv_rep = tv.repeat_interleave(G, dim=1).contiguous()
    cr = ca.cluster(tq, tk, cq, seed=w.cluster_seed, cluster_size_k=ck if ck != cq else 0)
    blocks = ca.route(cr.cent_q, cr.cent_k, 4)
    args = (cr.perm_q, cr.perm_k, cq, blocks)
    kw = dict(compensate=True, return_lse=True, fp8=fp8, c_k=ck)
    O, L = ca.attend(tq, tk, tv, *args, **kw)
    Or, Lr = ca.attend(tq, tk_rep, tv_rep, *args, **kw)
    assert torch.equal(O, Or) and torch.equal(L, Lr), (name, fp8)
    Krep, Vrep = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    Oo, Lo = o.attend(Q, Krep, Vrep, _np(cr.perm_q), _np(cr.perm_k), cq, _np(blocks), True,
                      c_k=ck, qk="e4m3" if fp8 else "exact")
    err, lerr = np.max(np.abs(_np(O) - Oo)), np.max(np.abs(_np(L) - Lo))
    tol = 2e-2 if dt == "bf16" else 1e-4
    print(f"{name} fp8={fp8}: max|O-oracle|={err:.2e} max|LSE-oracle|={lerr:.2e}")
    assert err <= tol and lerr <= (1e-2 if dt == "bf16" else 1e-4)


@pytest.mark.parametrize("split_mode", ["power", "diag"])
def test_shared_key_clustering(ca, split_mode):
    """kv_share: one key clustering per key/value head under the mean of its
    query heads' metrics (v1 §6.2, the first option). Every head of a group
    gets the same key permutation, centroids and counts; with identical query
    heads in a group of two (the mean of two equal fp32 metrics is exact) it
    equals the per-head clustering; against the oracle's shared trees the
    key clusters agree."""
    import torch
    w, Q, K, V, G, dt, cq, ck = _inputs("video_gqa4to2_bf16")
    tq, tk = _dev(Q, dt), _dev(K, dt)
    kw = dict(seed=w.cluster_seed, split_mode=split_mode)
    sh = ca.cluster(tq, tk, cq, kv_share=True, **kw)
    for g0 in range(0, Q.shape[1], G):
        for i in range(1, G):
            assert torch.equal(sh.perm_k[:, g0 + i], sh.perm_k[:, g0])
            assert torch.equal(sh.cent_k[:, g0 + i], sh.cent_k[:, g0])
            assert torch.equal(sh.counts[:, g0 + i], sh.counts[:, g0])
    # queries are clustered per head exactly as without sharing
    own = ca.cluster(tq, tk, cq, **kw)
    assert torch.equal(sh.perm_q, own.perm_q) and torch.equal(sh.cent_q, own.cent_q)
    # identical query heads within each group: the shared tree is the first head's own
    Qd = Q.copy()
    Qd[:, 1::2] = Qd[:, 0::2]
    tqd = _dev(Qd, dt)
    a = ca.cluster(tqd, tk, cq, kv_share=True, **kw)
    b = ca.cluster(tqd, tk, cq, **kw)
    assert torch.equal(a.perm_k[:, 0::2], b.perm_k[:, 0::2])
    if split_mode == "power":
        opts = o.ClusterOpts(seed=w.cluster_seed)
        Krep = np.repeat(K, G, axis=1)
        traces = {}
        _, pko = o.cluster(Q, Krep, cq, opts, dt, traces=traces, key_share=G)
        pk = _np(sh.perm_k)
        for h in range(0, Q.shape[1], G):
            ag, worst = check_tree(pk[0, h], pko[0, h], traces[(0, h, o.TENSOR_K)], Q.shape[2], cq,
                                   ("kv_share", h))
            print(f"shared key clusters, head {h}: agreement with the oracle {ag:.5f}, "
                  f"largest tie distance {worst:.2e} IQR")


@pytest.mark.parametrize("fp8", [False, True, "qkpv"])
@pytest.mark.parametrize("name", list(CASES))
def test_attend_kv_shared_equals_per_head(ca, name, fp8):
    """ca_attend_ex with kv_shared = 1 on a shared key clustering (every head
    of a group holds the same perm_k rows) builds the key tiles once per
    group and must give, bit for bit, the output and LSE of kv_shared = 0 on
    the same inputs (bf16 with query clusters of 128 and of 64, FP8 Q.K^T,
    FP8 P.V, fp32)."""
    import torch
    w, Q, K, V, G, dt, cq, ck = _inputs(name)
    if fp8 and dt != "bf16":
        pytest.skip("FP8 attention takes bf16 inputs")
    if fp8 == "qkpv" and cq < 128:
        pytest.skip("FP8 P.V needs query clusters of 128 or 256")
    tq, tk, tv = _dev(Q, dt), _dev(K, dt), _dev(V, dt)
    cr = ca.cluster(tq, tk, cq, seed=w.cluster_seed, cluster_size_k=ck if ck != cq else 0,
                    kv_share=True)
    blocks = ca.route(cr.cent_q, cr.cent_k, 4)
    for comp in (True, False):
        kw = dict(compensate=comp, return_lse=True, fp8=fp8, c_k=ck)
        O, L = ca.attend(tq, tk, tv, cr.perm_q, cr.perm_k, cq, blocks, kv_shared=True, **kw)
        Or, Lr = ca.attend(tq, tk, tv, cr.perm_q, cr.perm_k, cq, blocks, **kw)
        assert torch.equal(O, Or) and torch.equal(L, Lr), (name, fp8, comp)
