"""GPU parity of the FP8 (OCP E4M3) Q.K^T variant (dtype CA_BF16_FP8) and of
ca_quantize_e4m3. The pages run a quantized kernel and compare it with
quantized dense attention (paper "ClusterAttention: A training-free speedup
of bidirectional attention", arXiv 2608.26965 v1 §4.1 "Baselines"); the
group scheme is the oracle's stated reading.

Acceptance:

* ca_quantize_e4m3: codes and scales bit-exact against the oracle's
  quantize_e4m3 (bf16 and fp32 rows, per-row and 64-row groups, ragged last
  group, a dynamic range that reaches the subnormal codes, zero rows);
* lossless operands (every group's scale a power of two and every value on
  its group's grid): the FP8 path computes the bf16 path's logits up to fp32
  summation order, which can flip the bf16 rounding of a few P values (one
  flip moves the LSE by up to 2^-7 times that key's weight) and of outputs
  (one bf16 ulp: 2^-6 for values below 4), so outputs agree to 2e-2 and the
  LSE to 1e-2, while a key scale taken from the wrong sub-tile would move a
  tile's logits (of several units here) by a power of two;
* random operands: attention (top-k, ragged selection, query clusters
  smaller than key clusters, compensation on and off) and dense attention
  against the oracle with the same quantization: max-abs 2e-2 on O and 1e-2
  on the LSE, the bf16 path's bars; at the full video size on sampled query
  clusters of the GPU's own clusters.
"""
import math
import time

import numpy as np
import pytest

import oracle.clusterattn as o
import synth

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 2e-2, 1e-2


def _dev(x, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def _np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,D,group", [(1000, 128, 1), (1000, 128, 64), (777, 64, 64),
                                          (130, 12, 7), (3, 64, 1)])
def test_quantize_bit_exact(ca, dtype, rows, D, group):
    r = np.random.default_rng(rows * 7 + D + group)
    X = r.standard_normal((rows, D)) * np.exp2(r.integers(-20, 20, (rows, 1)))
    X[r.random((rows, D)) < 0.1] *= 2.0 ** -12          # subnormal codes and zeros
    X[0] = 0.0                                            # an all-zero row
    if rows > 2:
        X[1, :3] = [-0.0, 1e-30, -1e-30]
    X = X.astype(np.float32)
    if dtype == "bf16":
        X = synth.bf16_round(X)
    Xd = _dev(X, dtype)
    codes, scales = ca.quantize_e4m3(Xd, group)
    want_c, want_s = o.quantize_e4m3(_np(Xd).astype(np.float32), group)
    gc, gs = _np(codes), _np(scales)
    assert np.array_equal(gs.view(np.uint32), want_s.view(np.uint32)), (dtype, rows, D, group)
    bad = np.argwhere(gc != want_c)
    assert bad.size == 0, (dtype, rows, D, group, bad[:5], gc[tuple(bad[0])], want_c[tuple(bad[0])])


def _lossless_inputs(r, N, D, c, perm_k):
    """Q rows and 64-member key blocks of each cluster on power-of-two grids
    (one element +-448 * 2^(s-7) per row, the others e4m3 values at the same
    shift), shifts varying by row and by block."""
    def grid(n, shift):
        v = o.e4m3_decode(r.integers(0x20, 0x7F, (n, D))) * r.choice([-1.0, 1.0], (n, D))
        v[np.arange(n), r.integers(0, D, n)] = 448.0 * r.choice([-1.0, 1.0], n)
        return v * np.exp2(np.asarray(shift, np.float64) - 7.0).reshape(-1, 1)
    Q = grid(N, r.integers(-2, 1, N))
    K = np.empty((N, D))
    for j in range(-(-N // c)):
        mem = perm_k[j * c:(j + 1) * c]
        for p in range(0, len(mem), 64):
            K[mem[p:p + 64]] = grid(len(mem[p:p + 64]), r.integers(-2, 2))
    return Q.astype(np.float32), K.astype(np.float32)


@pytest.mark.parametrize("D,c", [(128, 128), (64, 64), (64, 256), (128, 256)])
def test_lossless_operands_match_bf16_path(ca, D, c):
    r = np.random.default_rng(D + c)
    N, H = 3000, 2
    nc = -(-N // c)
    topk = min(4, nc)
    pq = np.stack([r.permutation(N) for _ in range(H)])
    pk = np.stack([r.permutation(N) for _ in range(H)])
    Q = np.empty((1, H, N, D), np.float32); K = np.empty_like(Q)
    for h in range(H):
        Q[0, h], K[0, h] = _lossless_inputs(r, N, D, c, pk[h])
    V = r.standard_normal((1, H, N, D)).astype(np.float32)
    blocks = np.stack([np.stack([np.sort(r.choice(nc, topk, replace=False)) for _ in range(nc)])
                       for _ in range(H)])[None]
    tq, tk, tv = _dev(Q), _dev(K), _dev(V)
    args = (tq, tk, tv, _i32(pq[None]), _i32(pk[None]), c, _i32(blocks))
    O8, L8 = ca.attend(*args, compensate=False, return_lse=True, fp8=True)
    O16, L16 = ca.attend(*args, compensate=False, return_lse=True)
    eo, el = np.max(np.abs(_np(O8) - _np(O16))), np.max(np.abs(_np(L8) - _np(L16)))
    lo = o.sparse_attention(Q[0, 0], K[0, 0], V[0, 0], pq[0], pk[0], c, blocks[0, 0], False)[1]
    print(f"D={D} c={c}: fp8 vs bf16 path max|dO|={eo:.2e} max|dLSE|={el:.2e} "
          f"(LSE range {lo.min():.1f}..{lo.max():.1f})")
    assert eo <= 2e-2 and el <= 1e-2
    # dense: 64-token key blocks on one grid shift each
    Kd = np.empty_like(K)
    for h in range(H):
        Kd[0, h] = _lossless_inputs(r, N, D, 64, np.arange(N))[1]
    tkd = _dev(Kd)
    O8, L8 = ca.dense(tq, tkd, tv, return_lse=True, fp8=True)
    O16, L16 = ca.dense(tq, tkd, tv, return_lse=True)
    assert np.max(np.abs(_np(O8) - _np(O16))) <= 2e-2
    assert np.max(np.abs(_np(L8) - _np(L16))) <= 1e-2


CASES = {
    # name: (workload, N, heads, c_q, c_k, topk, ragged selection)
    "video_d128_c128_ragged": ("video_32760", 4000, 2, 128, 128, 4, False),
    "gmm_d64_c64": ("tabular_64k", 1500, 2, 64, 64, 5, False),
    "gmm_d64_c256_ragged": ("tabular_256k", 5000, 2, 256, 256, 3, False),
    "video_d128_q64_k128": ("video_32760", 4000, 2, 64, 128, 4, False),
    "peaked_d64_c128_adaptive": ("sweep_16k_peaked", 3000, 2, 128, 128, 0, True),
}


@pytest.mark.parametrize("compensate", [True, False])
@pytest.mark.parametrize("name", list(CASES))
def test_fp8_attend_against_oracle(ca, name, compensate):
    wname, N, H, cq, ck, topk, ragged = CASES[name]
    w = synth.WORKLOADS[wname]
    Q, K, V = synth.generate(w, heads=slice(0, H), N=N)
    B, _, _, D = Q.shape
    pq, pk = o.cluster(Q, K, cq, o.ClusterOpts(seed=w.cluster_seed), "bf16", c_k=ck)
    nq, nk = -(-N // cq), -(-N // ck)
    tau = 1.0 / math.sqrt(D)
    if ragged:
        blocks = np.full((B, H, nq, nk), -1, np.int32)
        nsel = np.zeros((B, H, nq), np.int32)
        sel = [[None] * H for _ in range(B)]
    else:
        blocks = np.empty((B, H, nq, topk), np.int32)
        nsel, sel = None, blocks
    for b in range(B):
        for h in range(H):
            cqm, _ = o.centroids(Q[b, h], pq[b, h], cq)
            ckm, cnt = o.centroids(K[b, h], pk[b, h], ck)
            if ragged:
                sel[b][h] = o.route_adaptive(cqm, ckm, cnt, tau, 0.9, 8)
                for a, s in enumerate(sel[b][h]):
                    blocks[b, h, a, :len(s)] = s
                    nsel[b, h, a] = len(s)
            else:
                blocks[b, h] = o.route(cqm, ckm, topk)
    O, L = ca.attend(_dev(Q), _dev(K), _dev(V), _i32(pq), _i32(pk), cq, _i32(blocks),
                     compensate=compensate, return_lse=True, fp8=True,
                     nsel=None if nsel is None else _i32(nsel), c_k=ck if ck != cq else 0)
    Oo, Lo = o.attend(Q, K, V, pq, pk, cq, sel, compensate, c_k=ck, qk="e4m3")
    Oe, Le = o.attend(Q, K, V, pq, pk, cq, sel, compensate, c_k=ck)
    err, lerr = np.max(np.abs(_np(O) - Oo)), np.max(np.abs(_np(L) - Lo))
    print(f"{name} comp={compensate}: max|O-oracle_fp8|={err:.2e} max|LSE-oracle_fp8|={lerr:.2e}; "
          f"fp8 vs exact oracle: max|dO|={np.max(np.abs(Oo - Oe)):.2e} "
          f"max|dLSE|={np.max(np.abs(Lo - Le)):.2e}")
    assert err <= TOL_O and lerr <= TOL_L, (name, compensate, err, lerr)


@pytest.mark.parametrize("name", ["video_d128_c128_ragged", "gmm_d64_c256_ragged"])
def test_fp8_dense_against_oracle(ca, name):
    wname, N, H = CASES[name][:3]
    w = synth.WORKLOADS[wname]
    Q, K, V = synth.generate(w, heads=slice(0, H), N=N)
    O, L = ca.dense(_dev(Q), _dev(K), _dev(V), return_lse=True, fp8=True)
    Oo, Lo = o.dense(Q, K, V, qk="e4m3")
    err, lerr = np.max(np.abs(_np(O) - Oo)), np.max(np.abs(_np(L) - Lo))
    print(f"{name} dense fp8: max|O-oracle_fp8|={err:.2e} max|LSE-oracle_fp8|={lerr:.2e}")
    assert err <= TOL_O and lerr <= TOL_L


def test_fp8_full_size_sampled(ca):
    """The video workload at full size as the bench runs it with --fp8: GPU
    clusters and routing, FP8 attention; sampled query clusters of two heads
    against the oracle on the GPU's clusters, and sampled rows of the FP8
    dense baseline."""
    import torch
    w = synth.WORKLOADS["video_32760"]
    heads = (0, 21)
    t0 = time.time()
    parts = [synth.generate(w, heads=slice(h, h + 1)) for h in range(w.H)]
    Q, K, V = (np.concatenate([p[i] for p in parts], axis=1) for i in range(3))
    print(f"inputs {Q.shape} in {time.time() - t0:.1f}s", flush=True)
    tq, tk, tv = _dev(Q), _dev(K), _dev(V)
    N, c, topk = w.N, w.c, w.topk
    res = ca.cluster(tq, tk, c, seed=w.cluster_seed)
    blocks = ca.route(res.cent_q, res.cent_k, topk)
    O, L = ca.attend(tq, tk, tv, res.perm_q, res.perm_k, c, blocks, compensate=w.compensate,
                     return_lse=True, fp8=True)
    Od, Ld = ca.dense(tq, tk, tv, return_lse=True, fp8=True)
    torch.cuda.synchronize()
    pq, pk, bl = _np(res.perm_q), _np(res.perm_k), _np(blocks)
    Og, Lg, Odg, Ldg = _np(O), _np(L), _np(Od), _np(Ld)
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(Odg))
    rng = np.random.default_rng(3)
    sizes = o.leaf_sizes(N, c)
    for h in heads:
        cl = np.sort(rng.choice(len(sizes), size=16, replace=False))
        Oo, Lo = o.sparse_attention(Q[0, h], K[0, h], V[0, h], pq[0, h], pk[0, h], c, bl[0, h],
                                    w.compensate, clusters=cl, qk="e4m3")
        rows = np.concatenate([pq[0, h][a * c:a * c + sizes[a]] for a in cl])
        err = np.max(np.abs(Og[0, h][rows] - Oo[rows]))
        lerr = np.max(np.abs(Lg[0, h][rows] - Lo[rows]))
        drows = np.sort(rng.choice(N, size=256, replace=False))
        Ood, Lod = o.dense_attention(Q[0, h][drows], K[0, h], V[0, h], qk="e4m3")
        derr = np.max(np.abs(Odg[0, h][drows] - Ood))
        dlerr = np.max(np.abs(Ldg[0, h][drows] - Lod))
        print(f"head {h}: sparse {len(rows)} rows max|O-oracle|={err:.2e} max|LSE-oracle|={lerr:.2e}; "
              f"dense 256 rows max|O-oracle|={derr:.2e} max|LSE-oracle|={dlerr:.2e}", flush=True)
        assert err <= TOL_O and lerr <= TOL_L and derr <= TOL_O and dlerr <= TOL_L


def test_zero_queries_and_key_blocks(ca):
    """Groups whose largest magnitude is 0 (scale 0): zero query rows and a
    whole key cluster of zero rows, including the short last cluster, so the
    masked keys of that tile meet a zero logit scale. Against the oracle,
    sparse and dense, compensation on."""
    w = synth.WORKLOADS["video_32760"]
    Q, K, V = synth.generate(w, heads=slice(0, 2), N=1000)
    B, H, N, D = Q.shape
    c, topk = 128, 3
    pq = np.stack([np.random.default_rng(h).permutation(N) for h in range(H)])[None]
    pk = np.stack([np.random.default_rng(10 + h).permutation(N) for h in range(H)])[None]
    Q[0, :, pq[0, 0, :40]] = 0.0                          # zero query rows
    nc = -(-N // c)
    for h in range(H):
        K[0, h, pk[0, h, 2 * c:3 * c]] = 0.0              # a full zero cluster
        K[0, h, pk[0, h, (nc - 1) * c:]] = 0.0            # the short last cluster
    blocks = np.stack([np.stack([np.array([0, 2, nc - 1]) for _ in range(nc)])
                       for _ in range(H)])[None].astype(np.int32)
    O, L = ca.attend(_dev(Q), _dev(K), _dev(V), _i32(pq), _i32(pk), c, _i32(blocks),
                     compensate=True, return_lse=True, fp8=True)
    Oo, Lo = o.attend(Q, K, V, pq, pk, c, blocks, True, qk="e4m3")
    assert np.all(np.isfinite(_np(O))) and np.all(np.isfinite(_np(L)))
    assert np.max(np.abs(_np(O) - Oo)) <= TOL_O and np.max(np.abs(_np(L) - Lo)) <= TOL_L
    Od, Ld = ca.dense(_dev(Q), _dev(K), _dev(V), return_lse=True, fp8=True)
    Odo, Ldo = o.dense(Q, K, V, qk="e4m3")
    assert np.max(np.abs(_np(Od) - Odo)) <= TOL_O and np.max(np.abs(_np(Ld) - Ldo)) <= TOL_L
