"""Seeded synthetic inputs for the ClusterAttention forward path.

This module only draws and shapes random numbers; it holds none of the
method's arithmetic. Both the HIP path (through tests and the bench) and the
CPU oracle (through tests) receive exactly the arrays produced here.

Every generator uses numpy's PCG64 (``np.random.default_rng(seed)``), draws in
float32 and, for bf16 workloads, rounds to bfloat16 with round-to-nearest-even.
The rounded values are returned as float32 arrays whose values are exactly
representable in bf16, so the GPU receives the same numbers the oracle widens
to fp64.

Workloads (shapes from the pages' experiments; the data itself is synthetic
because the models, datasets and prompts are not available):

* ``small_gmm_1k``      1 head, N=1024, d=64, fp32, c=64, top-4, compensation.
* ``tabular_64k``       8 heads, N=65536, d=64, bf16, c=128, top 1/8 (64).
* ``video_32760``       40 heads, N=32760 (21x30x52 latent grid), d=128, bf16,
                        c=128, top 1/8 (32).
* ``tabular_256k``      8 heads, N=262144, d=64, bf16, c=256, top 1/16 (64).
* ``sweep_16k``         16 heads, N=16384, d=64, bf16; peaked / flat regimes,
                        c in {64,128,256}, top fraction in {1/4,1/8,1/16}.

The tabular shapes follow the TabPFN-3 training-set sizes (about 93k-634k rows,
ClusterAttention arXiv v1 §4.2, Figure 2); the video shape is Wan 2.1-14B's
720p latent (§4.3).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_round", "bf16_bits", "generate",
    "gmm_qk", "video_qk", "flat_qk", "random_perm",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    r = ((b + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw 16-bit patterns of float32 values that are exact in bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not exactly representable in bfloat16")
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str            # "bf16" or "f32"
    c: int                # cluster size (queries and keys)
    topk: int             # selected key clusters per query cluster
    compensate: bool
    gen: str              # "gmm", "video", "flat", "peaked"
    components: int = 0   # mixture components for "gmm"/"peaked"
    data_seed: int = 0
    cluster_seed: int = 1
    control_seed: int = 2
    extra: dict = field(default_factory=dict)

    @property
    def n_c(self) -> int:
        return -(-self.N // self.c)


WORKLOADS = {
    "small_gmm_1k": Workload("small_gmm_1k", 1, 1, 1024, 64, "f32", 64, 4, True,
                             "gmm", 16, 1000, 1001, 1002),
    "tabular_64k": Workload("tabular_64k", 1, 8, 65536, 64, "bf16", 128, 64, True,
                            "gmm", 64, 2000, 2001, 2002),
    "video_32760": Workload("video_32760", 1, 40, 32760, 128, "bf16", 128, 32, True,
                            "video", 0, 3000, 3001, 3002),
    "tabular_256k": Workload("tabular_256k", 1, 8, 262144, 64, "bf16", 256, 64, True,
                             "gmm", 256, 4000, 4001, 4002),
    "sweep_16k_peaked": Workload("sweep_16k_peaked", 1, 16, 16384, 64, "bf16", 128, 16,
                                 True, "peaked", 64, 5000, 5001, 5002),
    "sweep_16k_flat": Workload("sweep_16k_flat", 1, 16, 16384, 64, "bf16", 128, 16,
                               True, "flat", 0, 5100, 5101, 5102),
}


def gmm_qk(rng: np.random.Generator, N: int, D: int, M: int, q_scale: float = 1.0):
    """One head of the anisotropic Gaussian-mixture queries and keys.

    Component means mu_m ~ 0.5 N(0, I) are shared by Q and K; each component has
    its own random mixing matrices A^Q_m, A^K_m ~ N(0,1)^{DxD}; token i draws a
    component z_i uniformly and q_i = mu_z + A^Q_z xi / sqrt(D),
    k_i = mu_z + A^K_z xi' / sqrt(D).
    """
    mu = 0.5 * rng.standard_normal((M, D), dtype=np.float32)
    AQ = rng.standard_normal((M, D, D), dtype=np.float32)
    AK = rng.standard_normal((M, D, D), dtype=np.float32)
    z = rng.integers(0, M, size=N)
    xq = rng.standard_normal((N, D), dtype=np.float32)
    xk = rng.standard_normal((N, D), dtype=np.float32)
    Q = np.empty((N, D), np.float32)
    K = np.empty((N, D), np.float32)
    inv = np.float32(1.0 / math.sqrt(D))
    for m in range(M):
        idx = np.nonzero(z == m)[0]
        if idx.size == 0:
            continue
        Q[idx] = mu[m] + (xq[idx] @ AQ[m].T) * inv
        K[idx] = mu[m] + (xk[idx] @ AK[m].T) * inv
    if q_scale != 1.0:
        Q *= np.float32(q_scale)
    return Q, K


def video_qk(rng: np.random.Generator, D: int, grid=(21, 30, 52), noise_var: float = 0.5):
    """One head of the smooth 3-D positional field with noise, tokens shuffled.

    p = (t/T, y/Y, x/X) over the latent grid; F ~ N(0, 2^2)^{Dx3},
    phi ~ U[0, 2pi); g(p) = sqrt(2) cos(2 pi F p + phi); Q = g + eps_Q,
    K = g + eps_K with eps ~ N(0, noise_var). The caller shuffles tokens.
    """
    T, Y, X = grid
    t, y, x = np.meshgrid(np.arange(T) / T, np.arange(Y) / Y, np.arange(X) / X,
                          indexing="ij")
    P = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float32)
    F = 2.0 * rng.standard_normal((D, 3), dtype=np.float32)
    phi = rng.uniform(0.0, 2.0 * math.pi, size=D).astype(np.float32)
    g = np.float32(math.sqrt(2.0)) * np.cos(np.float32(2.0 * math.pi) * (P @ F.T) + phi)
    sd = np.float32(math.sqrt(noise_var))
    Q = g + sd * rng.standard_normal(g.shape, dtype=np.float32)
    K = g + sd * rng.standard_normal(g.shape, dtype=np.float32)
    return Q.astype(np.float32), K.astype(np.float32)


def flat_qk(rng: np.random.Generator, N: int, D: int):
    """Isotropic queries and keys, N(0, I)."""
    return (rng.standard_normal((N, D), dtype=np.float32),
            rng.standard_normal((N, D), dtype=np.float32))


def generate(w: Workload, heads: slice | None = None, N: int | None = None):
    """Q, K, V of shape [B, H, N, D] (float32 values; bf16-exact for bf16).

    ``heads`` restricts generation to a subset of heads; every head has its own
    sub-stream keyed by (data_seed, b, h), so a subset equals the same slice of
    the full tensor. ``N`` overrides the token count (for small test cases of
    the same distribution; the video field keeps its grid and is truncated).
    """
    N = w.N if N is None else N
    hs = range(w.H)[heads] if heads is not None else range(w.H)
    Qs, Ks, Vs = [], [], []
    for b in range(w.B):
        qh, kh, vh = [], [], []
        for h in hs:
            rng = np.random.default_rng([w.data_seed, b, h])
            if w.gen == "gmm":
                Q, K = gmm_qk(rng, N, w.D, w.components)
            elif w.gen == "peaked":
                Q, K = gmm_qk(rng, N, w.D, w.components, q_scale=4.0)
            elif w.gen == "flat":
                Q, K = flat_qk(rng, N, w.D)
            elif w.gen == "video":
                Q, K = video_qk(rng, w.D)
                if N > Q.shape[0]:
                    raise ValueError("video field has at most %d tokens" % Q.shape[0])
                perm = rng.permutation(Q.shape[0])
                Q, K = Q[perm][:N], K[perm][:N]
            else:
                raise ValueError(w.gen)
            V = rng.standard_normal((N, w.D), dtype=np.float32)
            qh.append(Q); kh.append(K); vh.append(V)
        Qs.append(np.stack(qh)); Ks.append(np.stack(kh)); Vs.append(np.stack(vh))
    Q, K, V = np.stack(Qs), np.stack(Ks), np.stack(Vs)
    if w.dtype == "bf16":
        Q, K, V = bf16_round(Q), bf16_round(K), bf16_round(V)
    return Q, K, V


def random_perm(seed: int, B: int, H: int, N: int) -> np.ndarray:
    """Seeded random token permutations [B, H, N] (the random-cluster control)."""
    out = np.empty((B, H, N), np.int32)
    for b in range(B):
        for h in range(H):
            out[b, h] = np.random.default_rng([seed, b, h]).permutation(N)
    return out
