"""Python binding of the gfx950 ClusterAttention library (libca.so, include/ca.h).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI. PyTorch supplies device memory (outputs, workspace) and the
current HIP stream. The library must have been built in-tree
(``python -m free_clustered_block_amd.build``); nothing here falls back to a
CPU or framework implementation.

Paper: "ClusterAttention: A training-free speedup of bidirectional attention"
(arXiv 2608.26965).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "CAError", "load", "LIB_PATH", "EXPORTS", "profile_events", "peak_probe", "HipEvent", "tree_levels",
    "workspace_size", "cluster", "route", "route_noalloc", "route_adaptive", "attend", "dense", "forward",
    "quantize_e4m3",
    "ClusterResult",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libca.so")
EXPORTS = ["ca_tree_levels", "ca_workspace_size", "ca_cluster", "ca_route", "ca_route_noalloc",
           "ca_route_adaptive",
           "ca_attend", "ca_attend_var", "ca_attend_ex", "ca_dense", "ca_quantize_e4m3",
           "ca_profile_events", "ca_peak_probe", "ca_status_string", "ca_last_error"]

CA_BF16, CA_F32, CA_BF16_FP8, CA_BF16_FP8_PV = 0, 1, 2, 3
OP_CLUSTER, OP_ROUTE, OP_ATTEND, OP_DENSE, OP_CLUSTER_DIAG = 0, 1, 2, 3, 4

_lib = None


class CAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class _Opts(ctypes.Structure):
    _fields_ = [("transform", ctypes.c_int), ("query_normalize", ctypes.c_int),
                ("power_iters", ctypes.c_int), ("sample_factor", ctypes.c_int),
                ("seed", ctypes.c_uint64), ("trace_perm", ctypes.c_void_p),
                ("trace_score", ctypes.c_void_p), ("trace_dir", ctypes.c_void_p),
                ("split_mode", ctypes.c_int), ("trace_basis", ctypes.c_void_p),
                ("cluster_size_k", ctypes.c_int), ("kv_heads", ctypes.c_int),
                ("kv_share", ctypes.c_int)]

_SPLIT_MODES = {"power": 0, "diag": 1}


def load() -> ctypes.CDLL:
    """Load libca.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m free_clustered_block_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.ca_tree_levels.argtypes = [I, I]
    lib.ca_tree_levels.restype = I
    lib.ca_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.ca_workspace_size.restype = S
    lib.ca_cluster.argtypes = [P, P, I, I, I, I, I, I, ctypes.POINTER(_Opts), P, P, P, P, P, P, S, P]
    lib.ca_cluster.restype = I
    lib.ca_route.argtypes = [P, P, I, I, I, I, I, I, P, P, P, S, P]
    lib.ca_route.restype = I
    lib.ca_route_noalloc.argtypes = [P, P, I, I, I, I, I, I, P, P]
    lib.ca_route_noalloc.restype = I
    lib.ca_route_adaptive.argtypes = [P, P, P, I, I, I, I, I, F, F, I, P, P, P, P, S, P]
    lib.ca_route_adaptive.restype = I
    lib.ca_attend.argtypes = [P, P, P, I, I, I, I, I, P, P, I, P, I, I, F, P, P, P, S, P]
    lib.ca_attend.restype = I
    lib.ca_attend_var.argtypes = [P, P, P, I, I, I, I, I, P, P, I, P, P, I, I, F, P, P, P, S, P]
    lib.ca_attend_var.restype = I
    lib.ca_attend_ex.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, I, I, P, P, I, I, F, P, P, P, S, P]
    lib.ca_attend_ex.restype = I
    lib.ca_dense.argtypes = [P, P, P, I, I, I, I, I, F, P, P, P, S, P]
    lib.ca_dense.restype = I
    lib.ca_quantize_e4m3.argtypes = [P, I, ctypes.c_int64, I, I, P, P, P]
    lib.ca_quantize_e4m3.restype = I
    lib.ca_peak_probe.argtypes = [I, I, I, P, P]
    lib.ca_peak_probe.restype = I
    lib.ca_profile_events.argtypes = [P, P]
    lib.ca_profile_events.restype = I
    lib.ca_status_string.argtypes = [I]
    lib.ca_status_string.restype = ctypes.c_char_p
    lib.ca_last_error.argtypes = []
    lib.ca_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load()
        msg = lib.ca_status_string(status).decode()
        detail = lib.ca_last_error().decode()
        raise CAError(status, f"{msg}: {detail}")


def profile_events(start=None, stop=None) -> None:
    """Record two raw hipEvent_t handles (ints, see ``HipEvent``) around the
    attention kernel of the following attend/dense calls on this thread;
    None, None switches it off."""
    load().ca_profile_events(start, stop)


def peak_probe(kind: int, blocks: int, iters: int, out) -> None:
    """Launch the matrix-core (kind 0) or LDS (kind 1) peak-rate probe on the
    current stream; ``out`` is a float32 device tensor of blocks * 4 elements."""
    import torch
    if out.dtype != torch.float32 or out.numel() < blocks * 4 or not out.is_cuda:
        raise ValueError("out must be a float32 device tensor of at least blocks * 4 elements")
    _check(load().ca_peak_probe(kind, blocks, iters, out.data_ptr(), _stream_ptr(out.device)))


class HipEvent:
    """A raw timing hipEvent_t from the process's HIP runtime (the library
    records these itself, which torch.cuda.Event does not allow)."""
    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        self.handle = ctypes.c_void_p()
        if self._rt().hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        if self._rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.handle:
            self._hip.hipEventDestroy(self.handle)


def tree_levels(N: int, c: int) -> int:
    return load().ca_tree_levels(N, c)


def workspace_size(op: int, B: int, H: int, N: int, D: int, c: int = 0, topk: int = 0) -> int:
    return int(load().ca_workspace_size(op, B, H, N, D, c, topk))


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CA_BF16
    if t.dtype == torch.float32:
        return CA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(dev) -> int:
    torch = _torch()
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _ws(nbytes: int, dev, workspace=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None and workspace.numel() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _bhnd(*ts):
    for t in ts:
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("tensors must be contiguous [B, H, N, D] device tensors")


def _kv_heads(Q, *kv) -> int:
    """Head count of K (and V) when it differs from Q's (grouped- or
    multi-query attention), else 0."""
    B, H, N, D = Q.shape
    for t in kv:
        if t.shape[0] != B or t.shape[2:] != Q.shape[2:] or t.shape[1] != kv[0].shape[1]:
            raise ValueError("K and V must be [B, kv_heads, N, D] like Q")
    h = kv[0].shape[1]
    return 0 if h == H else h


@dataclass
class ClusterResult:
    perm_q: object
    perm_k: object
    cent_q: object
    cent_k: object
    counts: object
    trace_perm: object = None
    trace_score: object = None
    trace_dir: object = None
    trace_basis: object = None


def cluster(Q, K, c: int, *, transform: bool = True, query_normalize: bool = True,
            power_iters: int = 8, sample_factor: int = 1, seed: int = 0,
            split_mode: str = "power", cluster_size_k: int = 0, trace: bool = False,
            kv_share: bool = False, workspace=None) -> ClusterResult:
    """ca_cluster: permutations into clusters of size c and the cluster centroids.

    split_mode "power" is basic recursive splitting (power iteration per node),
    "diag" diagonalized recursive splitting (one principal-component basis per
    tree, each node splits along its highest-variance coordinate).
    cluster_size_k (0: c) clusters the keys with their own size. K may have
    fewer heads than Q (grouped- or multi-query attention): every query head
    then clusters its key/value head's rows under its own metric, or, with
    kv_share, each key/value head's keys are clustered once under the mean
    of its query heads' metrics (and copied to every head of the group)."""
    if split_mode not in _SPLIT_MODES:
        raise ValueError(f"split_mode must be one of {sorted(_SPLIT_MODES)}")
    torch = _torch()
    _bhnd(Q, K)
    B, H, N, D = Q.shape
    kvh = _kv_heads(Q, K)
    dev = Q.device
    ck = cluster_size_k or c
    n_c, n_kc = -(-N // c), -(-N // ck)
    perm_q = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    perm_k = torch.empty_like(perm_q)
    cent_q = torch.empty((B, H, n_c, D), dtype=torch.float32, device=dev)
    cent_k = torch.empty((B, H, n_kc, D), dtype=torch.float32, device=dev)
    counts = torch.empty((B, H, n_kc), dtype=torch.int32, device=dev)
    tp = ts = td = tb = None
    if trace:
        L = tree_levels(N, c)
        S = 1 << max(L - 1, 0)
        tp = torch.full((L + 1, B * H, 2, N), -1, dtype=torch.int32, device=dev)
        ts = torch.full((max(L, 1), B * H, 2, N), float("nan"), dtype=torch.float32, device=dev)
        td = torch.full((max(L, 1), B * H, 2, S, D), float("nan"), dtype=torch.float32, device=dev)
        if split_mode == "diag":
            tb = torch.full((B * H, 2, D, D), float("nan"), dtype=torch.float32, device=dev)
    opts = _Opts(int(transform), int(query_normalize), power_iters, sample_factor,
                 seed & ((1 << 64) - 1), _ptr(tp), _ptr(ts), _ptr(td),
                 _SPLIT_MODES[split_mode], _ptr(tb), int(cluster_size_k), kvh, int(kv_share))
    nbytes = workspace_size(OP_CLUSTER_DIAG if split_mode == "diag" else OP_CLUSTER, B, H, N, D,
                            min(c, ck))
    ws = _ws(nbytes, dev, workspace)
    st = load().ca_cluster(Q.data_ptr(), K.data_ptr(), _dtype_code(Q), B, H, N, D, c,
                           ctypes.byref(opts), perm_q.data_ptr(), perm_k.data_ptr(),
                           cent_q.data_ptr(), cent_k.data_ptr(), counts.data_ptr(),
                           _ptr(ws), nbytes, _stream_ptr(dev))
    _check(st)
    return ClusterResult(perm_q, perm_k, cent_q, cent_k, counts, tp, ts, td, tb)


def route(cent_q, cent_k, topk: int, *, return_scores: bool = False, workspace=None):
    """ca_route: top-k key clusters per query cluster (ascending indices)."""
    torch = _torch()
    B, H, nq, D = cent_q.shape
    nk = cent_k.shape[2]
    dev = cent_q.device
    blocks = torch.empty((B, H, nq, topk), dtype=torch.int32, device=dev)
    scores = torch.empty((B, H, nq, nk), dtype=torch.float32, device=dev) if return_scores else None
    nbytes = 0 if return_scores else workspace_size(OP_ROUTE, B, H, nq, D, nk, topk)
    ws = _ws(nbytes, dev, workspace)
    st = load().ca_route(cent_q.data_ptr(), cent_k.data_ptr(), B, H, nq, nk, D, topk,
                         blocks.data_ptr(), _ptr(scores), _ptr(ws), nbytes, _stream_ptr(dev))
    _check(st)
    return (blocks, scores) if return_scores else blocks


def route_noalloc(cent_q, cent_k, topk: int, *, blocks=None):
    """ca_route_noalloc: top-k key clusters per query cluster without a
    workspace (the library's scratch array holds the scores). ``blocks``, if
    given, is the int32 output tensor [B,H,n_qc,topk]; nothing is allocated
    then."""
    torch = _torch()
    B, H, nq, D = cent_q.shape
    nk = cent_k.shape[2]
    if blocks is None:
        blocks = torch.empty((B, H, nq, topk), dtype=torch.int32, device=cent_q.device)
    elif blocks.dtype != torch.int32 or tuple(blocks.shape) != (B, H, nq, topk) or not blocks.is_contiguous():
        raise ValueError("blocks must be a contiguous int32 tensor [B,H,n_qc,topk]")
    st = load().ca_route_noalloc(cent_q.data_ptr(), cent_k.data_ptr(), B, H, nq, nk, D, topk,
                                 blocks.data_ptr(), _stream_ptr(cent_q.device))
    _check(st)
    return blocks


def route_adaptive(cent_q, cent_k, counts_k, recall: float, *, min_count: int = 16,
                   scale: float = 0.0, return_scores: bool = False, workspace=None):
    """ca_route_adaptive: per query cluster the key clusters above a histogram
    cutoff that meets min_count and the estimated mass recall. Returns
    (blocks [B,H,n_qc,n_kc] with the first nsel entries of a row selected,
    nsel [B,H,n_qc]) and the scores if asked."""
    torch = _torch()
    B, H, nq, D = cent_q.shape
    nk = cent_k.shape[2]
    dev = cent_q.device
    blocks = torch.empty((B, H, nq, nk), dtype=torch.int32, device=dev)
    nsel = torch.empty((B, H, nq), dtype=torch.int32, device=dev)
    scores = torch.empty((B, H, nq, nk), dtype=torch.float32, device=dev) if return_scores else None
    nbytes = 0 if return_scores else workspace_size(OP_ROUTE, B, H, nq, D, nk, 1)
    ws = _ws(nbytes, dev, workspace)
    st = load().ca_route_adaptive(cent_q.data_ptr(), cent_k.data_ptr(), counts_k.data_ptr(), B, H,
                                  nq, nk, D, float(scale), float(recall), int(min_count),
                                  blocks.data_ptr(), nsel.data_ptr(), _ptr(scores), _ptr(ws),
                                  nbytes, _stream_ptr(dev))
    _check(st)
    return (blocks, nsel, scores) if return_scores else (blocks, nsel)


def _attn_dtype(Q, fp8) -> int:
    """fp8: False, True / "qk" (FP8 Q.K^T, CA_BF16_FP8) or "qkpv" (FP8 Q.K^T
    and P.V, CA_BF16_FP8_PV)."""
    dt = _dtype_code(Q)
    if fp8:
        if dt != CA_BF16:
            raise TypeError("fp8 attention takes bfloat16 inputs")
        if fp8 == "qkpv":
            return CA_BF16_FP8_PV
        if fp8 is True or fp8 == "qk":
            return CA_BF16_FP8
        raise ValueError("fp8 must be False, True, 'qk' or 'qkpv'")
    return dt


def attend(Q, K, V, perm_q, perm_k, c: int, blocks, *, compensate: bool = True,
           scale: float = 0.0, return_lse: bool = False, nsel=None, c_k: int = 0,
           fp8=False, kv_shared: bool = False, workspace=None):
    """ca_attend: block-sparse attention with optional mean-compensation;
    with `nsel` (selected count per row of `blocks`), ca_attend_var; with key
    clusters of another size c_k than the query clusters' c, or K and V with
    fewer heads than Q (grouped- or multi-query attention), ca_attend_ex;
    kv_shared=True (with fewer K/V heads): perm_k's rows are identical within
    each group of query heads (cluster(..., kv_share=True)), so the key tiles
    are built once per group; fp8=True (or "qk"): the Q.K^T product on FP8
    (E4M3) operands (dtype CA_BF16_FP8); fp8="qkpv": P.V on FP8 operands too
    (CA_BF16_FP8_PV)."""
    torch = _torch()
    _bhnd(Q, K, V)
    dt = _attn_dtype(Q, fp8)
    kvh = _kv_heads(Q, K, V)
    B, H, N, D = Q.shape
    dev = Q.device
    O = torch.empty_like(Q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    topk = blocks.shape[-1]
    ck = c_k or c
    nbytes = workspace_size(OP_ATTEND, B, H, N, D, ck, topk)
    ws = _ws(nbytes, dev, workspace)
    if ck != c or kvh:
        st = load().ca_attend_ex(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, kvh,
                                 int(bool(kv_shared)), N, D, perm_q.data_ptr(), perm_k.data_ptr(),
                                 c, ck, blocks.data_ptr(),
                                 _ptr(nsel), topk, int(compensate), float(scale), O.data_ptr(),
                                 _ptr(lse), _ptr(ws), nbytes, _stream_ptr(dev))
    elif nsel is None:
        st = load().ca_attend(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N, D,
                              perm_q.data_ptr(), perm_k.data_ptr(), c, blocks.data_ptr(), topk,
                              int(compensate), float(scale), O.data_ptr(), _ptr(lse), _ptr(ws),
                              nbytes, _stream_ptr(dev))
    else:
        st = load().ca_attend_var(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N,
                                  D, perm_q.data_ptr(), perm_k.data_ptr(), c, blocks.data_ptr(),
                                  nsel.data_ptr(), topk, int(compensate), float(scale),
                                  O.data_ptr(), _ptr(lse), _ptr(ws), nbytes, _stream_ptr(dev))
    _check(st)
    return (O, lse) if return_lse else O


def dense(Q, K, V, *, scale: float = 0.0, return_lse: bool = False, fp8=False,
          workspace=None):
    """ca_dense: dense attention baseline (fp8=True / "qk": FP8 Q.K^T operands;
    "qkpv": FP8 P.V operands too)."""
    torch = _torch()
    _bhnd(Q, K, V)
    if _kv_heads(Q, K, V):
        raise ValueError("dense() takes K and V with the head count of Q")
    dt = _attn_dtype(Q, fp8)
    B, H, N, D = Q.shape
    dev = Q.device
    O = torch.empty_like(Q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    nbytes = workspace_size(OP_DENSE, B, H, N, D)
    ws = _ws(nbytes, dev, workspace)
    st = load().ca_dense(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N, D,
                         float(scale), O.data_ptr(), _ptr(lse), _ptr(ws), nbytes, _stream_ptr(dev))
    _check(st)
    return (O, lse) if return_lse else O


def quantize_e4m3(X, group: int):
    """ca_quantize_e4m3: the rows of a 2-D bf16/fp32 tensor as FP8 (E4M3)
    codes (uint8, same shape) and one fp32 scale per `group` rows."""
    torch = _torch()
    if X.dim() != 2 or not X.is_contiguous():
        raise ValueError("X must be a contiguous 2-D tensor")
    R, D = X.shape
    codes = torch.empty((R, D), dtype=torch.uint8, device=X.device)
    scales = torch.empty(((R + group - 1) // group,), dtype=torch.float32, device=X.device)
    st = load().ca_quantize_e4m3(X.data_ptr(), _dtype_code(X), R, D, group, codes.data_ptr(),
                                 scales.data_ptr(), _stream_ptr(X.device))
    _check(st)
    return codes, scales


def forward(Q, K, V, c: int, topk: int, *, compensate: bool = True, seed: int = 0,
            return_all: bool = False, **cluster_kw):
    """The whole path: cluster -> route -> attend."""
    cr = cluster(Q, K, c, seed=seed, **cluster_kw)
    blocks = route(cr.cent_q, cr.cent_k, topk)
    O = attend(Q, K, V, cr.perm_q, cr.perm_k, c, blocks, compensate=compensate)
    return (O, cr, blocks) if return_all else O
