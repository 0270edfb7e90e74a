"""Pins of the oracle's FP8 (OCP E4M3) Q.K^T operands against the format's
definition, a library conversion, hand-worked values, lossless constructions
and the quantization error bound. The pages run a quantized kernel and compare
with quantized dense attention (paper "ClusterAttention: A training-free
speedup of bidirectional attention", arXiv 2608.26965 v1 §4.1 "Baselines");
the scheme itself is the oracle's stated reading. ``test_fp8_planted`` plants
plausible mistakes into the oracle (on the CPU) and requires a pin to fail.
"""
import math

import numpy as np
import pytest

import oracle.clusterattn as o


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# The E4M3 format
# ---------------------------------------------------------------------------

def check_e4m3_decode_library():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = o.e4m3_decode(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(got))
    fin = ~np.isnan(lib)
    assert np.array_equal(lib[fin], got[fin])
    # facts of the format: largest finite, smallest subnormal and normal, one
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.sum(np.isnan(got)) == 2


def check_e4m3_encode_library():
    import torch
    r = _rng(1)
    n = 100000
    x = np.exp2(r.uniform(-13.0, 8.9, n)) * r.choice([-1.0, 1.0], n)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3_encode(x), lib)
    # every finite code round-trips; midpoints go to the even code
    codes = np.arange(256, dtype=np.uint8)
    vals = o.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(o.e4m3_encode(vals[fin]), codes[fin])
    for c in range(0, 0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert o.e4m3_encode(mid) == even, c
        assert o.e4m3_encode(np.nextafter(mid, 0.0)) == c
        assert o.e4m3_encode(np.nextafter(mid, 1e9)) == c + 1
        assert o.e4m3_encode(-mid) == (even | 0x80)
    # saturation above the largest finite value and the sign of zero
    assert o.e4m3_encode(500.0) == 0x7E and o.e4m3_encode(-1e6) == 0xFE
    assert o.e4m3_encode(0.0) == 0x00 and o.e4m3_encode(-0.0) == 0x80


def check_bf16_library():
    import torch
    r = _rng(2)
    x = (r.standard_normal(50000) * np.exp2(r.uniform(-20, 20, 50000))).astype(np.float32)
    lib = torch.from_numpy(x).bfloat16().float().numpy()
    assert np.array_equal(o.bf16_nearest(x), lib)


# ---------------------------------------------------------------------------
# Group quantization
# ---------------------------------------------------------------------------

def check_quantize_worked_example():
    # amax 1: inv = 448; 1 -> 448 (0x7E); -0.5 -> -224 = -1.75 * 2^7 (0xF6);
    # fp32(0.3 * 448) = 134.4 lies in [128, 256), spacing 16 -> 128 (0x70)
    codes, scales = o.quantize_e4m3(np.array([[1.0, -0.5, 0.3]], np.float32), 1)
    assert codes.tolist() == [[0x7E, 0xF6, 0x70]]
    assert scales.dtype == np.float32 and scales[0] == np.float32(1.0) / np.float32(448.0)
    # a group of two rows shares one scale; an all-zero group: codes 0, scale 0
    X = np.array([[2.0, 0.0], [0.0, -1.0], [0.0, 0.0]], np.float32)
    codes, scales = o.quantize_e4m3(X, 2)
    assert codes.tolist() == [[0x7E, 0x00], [0x00, 0xF6], [0x00, 0x00]]
    assert scales.tolist() == [np.float32(2.0) / np.float32(448.0), 0.0]


def check_quantize_bounds():
    r = _rng(3)
    for R, D, g in [(200, 64, 1), (200, 64, 64), (131, 128, 64), (5, 8, 7)]:
        X = (r.standard_normal((R, D)) * np.exp2(r.integers(-8, 8, (R, 1)))).astype(np.float32)
        X[r.random((R, D)) < 0.05] *= 1e-4          # values in the subnormal range
        codes, scales = o.quantize_e4m3(X, g)
        assert codes.shape == X.shape and scales.shape == ((R + g - 1) // g,)
        Xh = o.dequantize_e4m3(codes, scales, g)
        for k in range(len(scales)):
            blk = slice(k * g, (k + 1) * g)
            amax = np.abs(X[blk]).max()
            # the group's largest magnitude maps to the largest code
            assert np.abs(o.e4m3_decode(codes[blk])).max() == 448.0
            assert abs(float(scales[k]) * 448.0 - amax) <= 2 * np.spacing(np.float32(amax))
            # error: half a spacing, 2^-4 relative in the normal range, 2^-10
            # code units below it, plus the fp32 rounding of the scales
            err = np.abs(Xh[blk] - X[blk])
            bound = np.maximum(2.0 ** -4 * np.abs(X[blk]), 2.0 ** -10 * scales[k]) * (1 + 1e-6) \
                + 1e-6 * np.abs(X[blk])
            assert np.all(err <= bound)


# ---------------------------------------------------------------------------
# FP8 attention
# ---------------------------------------------------------------------------

def _grid_rows(r, n, D, shift):
    """Rows of e4m3 code values times 2^(shift - 7), each with one element
    +-448: a group's amax is then 3.5 * 2^max(shift), its scale a power of two
    and its quantization exact; magnitudes >= 2^-3 keep shifts of a few
    binades inside a group in the normal range."""
    codes = r.integers(0x18, 0x7F, (n, D))            # 2^-3 .. 448
    vals = o.e4m3_decode(codes) * r.choice([-1.0, 1.0], (n, D))
    vals[np.arange(n), r.integers(0, D, n)] = 448.0 * r.choice([-1.0, 1.0], n)
    return vals * np.exp2(np.asarray(shift, np.float64) - 7.0)[..., None] \
        if np.ndim(shift) else vals * 2.0 ** (shift - 7)


def check_fp8_attention_lossless():
    """Operands that every group quantizes exactly: FP8 attention equals the
    exact one. The two 64-member halves of each 128-key cluster lie 2^12
    apart in magnitude, and so do the clusters, so a grouping other than per
    64 members of a cluster, or per-tensor query scaling, loses precision."""
    r = _rng(4)
    N, D, c = 640, 16, 128
    nc = N // c
    perm_q = r.permutation(N)
    perm_k = r.permutation(N)
    Q = np.empty((N, D)); K = np.empty((N, D))
    Q[:] = _grid_rows(r, N, D, r.integers(-6, 7, N))
    for j in range(nc):
        for half in range(2):
            K[perm_k[j * c + 64 * half:j * c + 64 * half + 64]] = \
                _grid_rows(r, 64, D, 12 * half + 3 * j - 12)
    V = r.standard_normal((N, D))
    blocks = np.array([np.sort(r.choice(nc, 2, replace=False)) for _ in range(nc)])
    a = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, False, qk="e4m3")
    b = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, False)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], rtol=0, atol=1e-9)
    # compensation: identical rows within a cluster make every centroid a
    # grid row, and close cluster magnitudes keep the centroid blocks exact
    for j in range(nc):
        K[perm_k[j * c:(j + 1) * c]] = _grid_rows(r, 1, D, j % 3 - 1)
    a = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, True, qk="e4m3")
    b = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, True)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], rtol=0, atol=1e-9)
    # dense: key blocks of 64 consecutive tokens, 2^3 apart
    Kd = np.concatenate([_grid_rows(r, 64, D, 3 * j - 12) for j in range(N // 64)])
    a = o.dense_attention(Q, Kd, V, qk="e4m3")
    b = o.dense_attention(Q, Kd, V)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], rtol=0, atol=1e-9)


def check_fp8_centroid_double_rounding():
    """Worked example: the excluded cluster's centroid (3.5, x) with
    x = (1.0625 + 2^-12) / 128 rounds to bf16 (1.0625) / 128, then to the
    even e4m3 code 1.0 (scale 3.5 / 448 = 2^-7), giving x_hat = 2^-7; the
    query (3.5, 3.5) is exact. Each query sees 64 keys (3.5, 0) and the
    centroid with weight 64: LSE = ln(64 e^(12.25 t) + 64 e^((12.25 +
    3.5 * 2^-7) t)), t = 1 / sqrt(2)."""
    N, D, c = 128, 2, 64
    x = (1.0625 + 2.0 ** -12) / 128
    Q = np.full((N, D), 3.5)
    K = np.zeros((N, D)); K[:, 0] = 3.5; K[64:, 1] = x
    V = np.zeros((N, D))
    perm = np.arange(N)
    blocks = np.zeros((2, 1), np.int64)
    _, L = o.sparse_attention(Q, K, V, perm, perm, c, blocks, True, qk="e4m3")
    t = 1.0 / math.sqrt(2.0)
    want = math.log(64 * math.exp(12.25 * t) + 64 * math.exp((12.25 + 3.5 * 2.0 ** -7) * t))
    assert np.allclose(L, want, rtol=0, atol=1e-12)


def check_fp8_attention_error_bound():
    """Random operands: every FP8 logit is within the bound that the group
    spacings give of the exact logit, so the LSE moves by no more than the
    largest logit error of its row."""
    r = _rng(5)
    N, D, c = 256, 32, 64
    Q = r.standard_normal((N, D)); K = r.standard_normal((N, D)) + 0.5; V = r.standard_normal((N, D))
    Q = Q.astype(np.float32).astype(np.float64); K = K.astype(np.float32).astype(np.float64)
    perm_q = r.permutation(N); perm_k = r.permutation(N)
    nc = N // c
    blocks = np.array([np.sort(r.choice(nc, 2, replace=False)) for _ in range(nc)])
    tau = 1.0 / math.sqrt(D)
    a = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, False, qk="e4m3")
    b = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, False)
    sq = np.abs(Q).max(axis=1) / 448.0
    sk = np.empty(N)
    for j in range(nc):
        mem = perm_k[j * c:(j + 1) * c]
        sk[mem] = np.abs(K[mem]).max() / 448.0
    eq = np.maximum(2.0 ** -4 * np.abs(Q), 2.0 ** -10 * sq[:, None]) * 1.001   # |q_hat - q|
    ek = np.maximum(2.0 ** -4 * np.abs(K), 2.0 ** -10 * sk[:, None]) * 1.001
    bound = tau * (eq @ (np.abs(K) + ek).T + np.abs(Q) @ ek.T)                  # [query, key]
    for qa in range(nc):
        qi = perm_q[qa * c:(qa + 1) * c]
        keys = np.concatenate([perm_k[j * c:(j + 1) * c] for j in blocks[qa]])
        lim = bound[np.ix_(qi, keys)].max(axis=1)
        assert np.all(np.abs(a[1][qi] - b[1][qi]) <= lim)
    # and the quantized result really differs from the exact one
    assert np.max(np.abs(a[1] - b[1])) > 1e-6


# ---------------------------------------------------------------------------
# FP8 value operands (P.V): power-of-two scales per dimension and 32 members
# ---------------------------------------------------------------------------

def check_e8m0_bruteforce():
    """The scale exponent is the smallest e with amax <= 448 * 2^e (searched
    directly), floored at -127, and 0 for an all-zero group."""
    r = _rng(6)
    vals = np.concatenate([np.exp2(r.uniform(-140.0, 120.0, 4000)),
                           448.0 * np.exp2(np.arange(-130, 100, dtype=np.float64)),
                           np.nextafter(448.0 * np.exp2(np.arange(-20, 20.0)), np.inf),
                           np.array([1.0, 3.0, 224.0, 448.0, 449.0, 2.0 ** -149])])
    for a in vals:
        e = -200
        while a > 448.0 * 2.0 ** e:
            e += 1
        assert o.e8m0_exponent(a) == max(e, -127), a
    assert o.e8m0_exponent(0.0) == 0


def check_mx_quantize_worked_example():
    # amax 3: e = -7 (448 * 2^-7 = 3.5 >= 3 > 1.75); 3 * 128 = 384 = 1.5 * 2^8 (0x7C);
    # 0.3 * 128 = 38.4 in [32, 64), spacing 4 -> 40 (0x62), i.e. 0.3125; -128 (0xF0)
    X = np.array([[3.0, 0.0], [0.3, 0.0], [-1.0, 0.0]])
    codes, expo = o.quantize_mx_e4m3(X, 32)
    assert codes[:, 0].tolist() == [0x7C, 0x62, 0xF0] and codes[:, 1].tolist() == [0, 0, 0]
    assert expo.tolist() == [[-7, 0]]
    assert o.fp8_value_rows(X, 32)[:, 0].tolist() == [3.0, 0.3125, -1.0]
    # two groups of two rows: per column and per group
    Y = np.array([[1.0, 448.0], [-2.0, 1.0], [0.25, 0.0], [0.0, 900.0]])
    codes, expo = o.quantize_mx_e4m3(Y, 2)
    assert expo.tolist() == [[-7, 0], [-10, 2]]


def check_mx_quantize_bounds():
    r = _rng(7)
    for R, D, g in [(256, 64, 32), (100, 16, 32), (33, 8, 32), (64, 4, 7)]:
        X = r.standard_normal((R, D)) * np.exp2(r.integers(-10, 10, (1, D)))
        X[r.random((R, D)) < 0.05] *= 1e-4
        codes, expo = o.quantize_mx_e4m3(X, g)
        Xh = o.fp8_value_rows(X, g)
        for k in range(expo.shape[0]):
            blk = slice(k * g, (k + 1) * g)
            amax = np.abs(X[blk]).max(axis=0)
            sc = np.exp2(expo[k].astype(np.float64))
            # the group's largest magnitude lands in (224, 448] code units
            assert np.all((amax / sc > 224.0) & (amax / sc <= 448.0))
            err = np.abs(Xh[blk] - X[blk])
            assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(X[blk]), 2.0 ** -10 * sc))


def _value_grid(r, n, D, shift):
    """Rows of e4m3 code values times 2^(shift - 7): every per-dimension group
    with a fixed shift quantizes exactly under a power-of-two scale."""
    codes = r.integers(0x18, 0x7F, (n, D))
    vals = o.e4m3_decode(codes) * r.choice([-1.0, 1.0], (n, D))
    return vals * 2.0 ** (shift - 7)


def check_fp8_values_lossless():
    """Values that every group (one dimension, 32 consecutive members of a
    cluster) quantizes exactly give the exact attention. The two 32-member
    halves of each 64-member block, the dimensions and the clusters lie 2^12
    apart, so per-64-member, per-token or token-order grouping loses
    precision."""
    r = _rng(8)
    N, D, c = 512, 8, 128
    nc = N // c
    perm_q = r.permutation(N); perm_k = r.permutation(N)
    Q = r.standard_normal((N, D)); K = r.standard_normal((N, D))
    V = np.empty((N, D))
    dshift = 12 * (np.arange(D) % 3) - 12
    for j in range(nc):
        for b in range(c // 32):
            mem = perm_k[j * c + 32 * b:j * c + 32 * b + 32]
            V[mem] = _value_grid(r, 32, D, 0) * np.exp2(dshift + 12.0 * (b % 2) + j)[None, :]
    blocks = np.array([np.sort(r.choice(nc, 2, replace=False)) for _ in range(nc)])
    assert np.array_equal(o.fp8_values(V, perm_k, c), V)
    a = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, False, pv="e4m3")
    b = o.sparse_attention(Q, K, V, perm_q, perm_k, c, blocks, False)
    assert np.allclose(a[0], b[0], rtol=1e-13, atol=0) and np.array_equal(a[1], b[1])
    # dense: groups of 32 consecutive tokens
    Vd = np.concatenate([_value_grid(r, 32, D, 0) * np.exp2(dshift + 12.0 * (k % 2))[None, :]
                         for k in range(N // 32)])
    a = o.dense_attention(Q, K, Vd, pv="e4m3")
    b = o.dense_attention(Q, K, Vd)
    assert np.allclose(a[0], b[0], rtol=1e-13, atol=0)


def check_fp8_value_centroid_double_rounding():
    """Worked example: the excluded cluster's value centroid x = (1.0625 +
    2^-12) / 128 rounds to bf16 (1.0625 / 128); its group (32 centroids, the
    others 0) has amax 1.0625 / 128, e = -15 (448 * 2^-15 = 0.0137 >= x), and
    x * 2^15 = 272 is the midpoint of the codes 256 and 288, so it rounds to
    the even 256: x_hat = 2^-7. With the selected cluster's values 0 and
    weights 64 : 64 e^0, the output is x_hat / 2 = 2^-8 (without the bf16
    rounding, 272.0625 would round up to 288)."""
    N, D, c = 128, 1, 64
    x = (1.0625 + 2.0 ** -12) / 128
    Q = np.zeros((N, D)); K = np.zeros((N, D))
    V = np.zeros((N, D)); V[64:, 0] = x
    perm = np.arange(N)
    blocks = np.array([[0], [0]])
    O, _ = o.sparse_attention(Q, K, V, perm, perm, c, blocks, True, pv="e4m3")
    assert np.allclose(O[:, 0], 2.0 ** -8, rtol=0, atol=1e-15)
    Oe, _ = o.sparse_attention(Q, K, V, perm, perm, c, blocks, True)
    assert abs(Oe[0, 0] - x / 2) < 1e-15 and abs(Oe[0, 0] - O[0, 0]) > 1e-7


def check_pv_rounding_bound():
    """The bound tests/fp8_bound.py gives holds for the kernel's algorithm run
    in fp64: sub-tiles of 64 terms, a running maximum that moves only when a
    sub-tile's maximum exceeds it by more than 8 (log2 units), weights
    2^(l - m) rounded to E4M3, accumulators rescaled when m moves, the
    denominator over the unrounded weights. And the rounding is visible."""
    from fp8_bound import pv_rounding_bound
    r = _rng(9)
    worst = 0.0
    for trial in range(40):
        T, D = int(r.integers(64, 600)), 8
        spread = [0.5, 3.0, 12.0][trial % 3]
        L2 = r.standard_normal((4, T)) * spread + r.standard_normal((4, 1)) * 20   # log2 units
        Vh = o.fp8_value_rows(r.standard_normal((T, D)), 32)
        want = (np.exp2(L2 - L2.max(1, keepdims=True)) @ Vh) / np.exp2(
            L2 - L2.max(1, keepdims=True)).sum(1, keepdims=True)
        for i in range(4):
            m, acc, den = -np.inf, np.zeros(D), 0.0
            for t0 in range(0, T, 64):
                blk = L2[i, t0:t0 + 64]
                bm = blk.max()
                if bm > m + 8:
                    alpha = np.exp2(m - bm) if m > -np.inf else 0.0
                    acc, den, m = acc * alpha, den * alpha, bm
                P = np.exp2(blk - m)
                assert P.max() <= 256.0
                Ph = o.e4m3_decode(o.e4m3_encode(P))
                acc = acc + Ph @ Vh[t0:t0 + 64]
                den += P.sum()
            got = acc / den
            b = pv_rounding_bound(L2[i:i + 1] * np.log(2.0), Vh)[0]
            assert np.all(np.abs(got - want[i]) <= b * (1 + 1e-9) + 1e-12)
            worst = max(worst, float(np.max(np.abs(got - want[i]))))
    assert worst > 1e-4


CHECKS = [check_e4m3_decode_library, check_e4m3_encode_library, check_bf16_library,
          check_quantize_worked_example, check_quantize_bounds, check_fp8_attention_lossless,
          check_fp8_centroid_double_rounding, check_fp8_attention_error_bound,
          check_e8m0_bruteforce, check_mx_quantize_worked_example, check_mx_quantize_bounds,
          check_fp8_values_lossless, check_fp8_value_centroid_double_rounding,
          check_pv_rounding_bound]


@pytest.mark.parametrize("check", CHECKS, ids=[f.__name__ for f in CHECKS])
def test_fp8_pin(check):
    check()


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

_orig = {n: getattr(o, n) for n in ("e4m3_encode", "fp8_keys", "fp8_rows", "fp8_centroids",
                                    "quantize_e4m3", "bf16_nearest", "e8m0_exponent",
                                    "fp8_values", "fp8_value_rows", "fp8_value_centroids")}


def _encode_truncating(x):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    q = np.exp2(np.maximum(ex - 1, -6) - 3.0)
    return _orig["e4m3_encode"](np.copysign(np.floor(a / q) * q, x))


def _encode_no_subnormals(x):
    x = np.asarray(x, np.float64)
    return _orig["e4m3_encode"](np.where(np.abs(x) < 2.0 ** -6, 0.0 * x, x))


def _keys_token_order(K, perm_k, ck, tile=64):
    return _orig["fp8_keys"](K, np.arange(np.shape(K)[0]), ck, tile)


def _keys_per_cluster(K, perm_k, ck, tile=64):
    return _orig["fp8_keys"](K, perm_k, ck, ck)


def _rows_per_tensor(X, group):
    return _orig["fp8_rows"](X, np.shape(X)[0])


def _centroids_without_bf16(kbar, tile=64):
    return _orig["fp8_rows"](np.asarray(kbar, np.float32), tile)


def _quantize_scale_from_inverse(X, group):
    codes, scales = _orig["quantize_e4m3"](X, group)
    inv = np.where(scales > 0, np.float32(448.0) / (scales * np.float32(448.0)), 0)
    return codes, np.where(scales > 0, np.float32(1.0) / inv.astype(np.float32) * np.float32(1.001), 0
                           ).astype(np.float32)


def _e8m0_one_too_low(amax):
    e = _orig["e8m0_exponent"](amax)
    return e - 1 if amax > 0 else e


def _values_per_64(V, perm_k, ck, block=32):
    return _orig["fp8_values"](V, perm_k, ck, 64)


def _values_token_order(V, perm_k, ck, block=32):
    return _orig["fp8_values"](V, np.arange(np.shape(V)[0]), ck, block)


def _value_rows_not_power_of_two(X, block):
    X = np.asarray(X, np.float64)
    out = np.empty_like(X)
    for g in range(0, X.shape[0], block):
        blk = X[g:g + block]
        amax = np.abs(blk).max(axis=0)
        sc = np.where(amax > 0, amax / 448.0, 1.0)
        out[g:g + block] = o.e4m3_decode(o.e4m3_encode(blk / sc)) * sc
    return out


def _value_rows_per_token(X, block):
    return _orig["fp8_value_rows"](np.asarray(X).T, np.shape(X)[1]).T


def _value_centroids_without_bf16(vbar, block=32):
    return _orig["fp8_value_rows"](np.asarray(vbar, np.float64), block)


PLANTED = [
    ("e8m0_exponent", _e8m0_one_too_low, check_e8m0_bruteforce),
    ("fp8_values", _values_per_64, check_fp8_values_lossless),
    ("fp8_values", _values_token_order, check_fp8_values_lossless),
    ("fp8_value_rows", _value_rows_not_power_of_two, check_fp8_values_lossless),
    ("fp8_value_rows", _value_rows_per_token, check_fp8_values_lossless),
    ("fp8_value_centroids", _value_centroids_without_bf16, check_fp8_value_centroid_double_rounding),
    ("e4m3_encode", _encode_truncating, check_e4m3_encode_library),
    ("e4m3_encode", _encode_no_subnormals, check_e4m3_encode_library),
    ("fp8_keys", _keys_token_order, check_fp8_attention_lossless),
    ("fp8_keys", _keys_per_cluster, check_fp8_attention_lossless),
    ("fp8_rows", _rows_per_tensor, check_fp8_attention_lossless),
    ("fp8_centroids", _centroids_without_bf16, check_fp8_centroid_double_rounding),
    ("quantize_e4m3", _quantize_scale_from_inverse, check_quantize_bounds),
]


def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,mutant,check", PLANTED,
                         ids=[f"{p[0]}-{p[1].__name__.lstrip('_')}" for p in PLANTED])
def test_fp8_planted(monkeypatch, name, mutant, check):
    check()
    monkeypatch.setattr(o, name, mutant)
    assert _fails(check), f"planted mistake in {name} was not caught"
