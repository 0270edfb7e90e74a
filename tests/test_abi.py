"""C-ABI checks that run without a GPU: the library loads, exports every
symbol include/ca.h declares, lays out the same tree as the oracle, sizes its
workspace, and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

import oracle.clusterattn as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ca.h")


@pytest.fixture(scope="module")
def lib():
    import free_clustered_block_amd as ca
    return ca.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ca_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    import free_clustered_block_amd as ca
    names = declared_functions()
    assert set(names) == set(ca.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_tree_levels_match_oracle(lib):
    for N, c in [(1024, 64), (65536, 128), (32760, 128), (262144, 256), (16384, 64),
                 (1000, 64), (64, 64), (65, 64), (3 * 64, 64), (7 * 128 + 5, 128)]:
        levels = o.tree_levels(N, c)
        want = sum(1 for lv in levels if any(nd.n > c for nd in lv))
        assert lib.ca_tree_levels(N, c) == want, (N, c)
    assert lib.ca_tree_levels(0, 64) == -1


def test_workspace_sizes(lib):
    import free_clustered_block_amd as ca
    SIZE_MAX = 2**64 - 1
    for op in (ca.OP_CLUSTER, ca.OP_ATTEND, ca.OP_DENSE):
        n = ca.workspace_size(op, 1, 8, 65536, 64, 128, 64)
        assert 0 < n < 2**40 and n % 256 == 0
    assert ca.workspace_size(ca.OP_ROUTE, 1, 8, 512, 64, 512, 64) == 8 * 512 * 512 * 4
    # the diagonalized split adds the coordinates of every vector: 2 B H N D floats
    extra = (ca.workspace_size(ca.OP_CLUSTER_DIAG, 1, 8, 65536, 64, 128, 64)
             - ca.workspace_size(ca.OP_CLUSTER, 1, 8, 65536, 64, 128, 64))
    assert 2 * 8 * 65536 * 64 * 4 <= extra < 2 * 8 * 65536 * 64 * 4 + 512
    assert ca.workspace_size(ca.OP_CLUSTER, 1, 1, 10, 64, 64, 1) == SIZE_MAX
    assert ca.workspace_size(ca.OP_ATTEND, 0, 1, 1024, 64, 64, 1) == SIZE_MAX


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def _cluster(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, dt=0, B=1, H=1, N=1024, D=64, c=64, opts=None, pq=FAKE, pk=FAKE,
             cq=FAKE, ck=FAKE, counts=None, ws=FAKE, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.ca_cluster(a["Q"], a["K"], a["dt"], a["B"], a["H"], a["N"], a["D"], a["c"], a["opts"],
                          a["pq"], a["pk"], a["cq"], a["ck"], a["counts"], a["ws"], a["ws_bytes"],
                          a["stream"])


def _attend(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=0, B=1, H=1, N=1024, D=64, pq=FAKE, pk=FAKE, c=64,
             blocks=FAKE, topk=4, comp=1, scale=0.0, O=FAKE, lse=None, ws=FAKE, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.ca_attend(a["Q"], a["K"], a["V"], a["dt"], a["B"], a["H"], a["N"], a["D"], a["pq"],
                         a["pk"], a["c"], a["blocks"], a["topk"], a["comp"], a["scale"], a["O"],
                         a["lse"], a["ws"], a["ws_bytes"], a["stream"])


def test_cluster_rejects_bad_arguments(lib):
    import free_clustered_block_amd as ca
    assert _cluster(lib, Q=None) == 1
    assert _cluster(lib, dt=7) == 1
    assert _cluster(lib, D=96) == 2
    assert _cluster(lib, c=100) == 2
    assert _cluster(lib, N=32) == 1
    assert _cluster(lib, B=0) == 1
    assert _cluster(lib, B=2**16, H=2**16) == 2
    opts = ca._Opts(1, 1, 0, 1, 0, None, None, None)
    assert _cluster(lib, opts=ctypes.byref(opts)) == 1
    opts = ca._Opts(1, 1, 8, 0, 0, None, None, None)
    assert _cluster(lib, opts=ctypes.byref(opts)) == 1
    opts = ca._Opts(1, 1, 8, 1, 0, None, None, None, 2, None)
    assert _cluster(lib, opts=ctypes.byref(opts)) == 1
    assert b"split_mode" in lib.ca_last_error()
    assert _cluster(lib, ws=None, ws_bytes=0) == 3
    assert _cluster(lib, ws=FAKE + 8, ws_bytes=2**30) == 3
    assert _cluster(lib, ws_bytes=100) == 3
    assert b"workspace" in lib.ca_last_error()
    assert lib.ca_status_string(3) == b"workspace missing, misaligned or too small"


def test_attend_rejects_bad_arguments(lib):
    assert _attend(lib, blocks=None) == 1
    assert _attend(lib, topk=0) == 1
    assert _attend(lib, topk=17) == 1          # n_c = 16
    assert _attend(lib, scale=-1.0) == 1
    assert _attend(lib, scale=float("nan")) == 1
    assert _attend(lib, scale=1e-35) == 1          # compensation carries ln n_c / scale
    assert _attend(lib, D=32) == 2
    assert _attend(lib, c=32) == 2
    assert _attend(lib, ws_bytes=10) == 3


def test_route_and_dense_reject_bad_arguments(lib):
    assert lib.ca_route(FAKE, FAKE, 1, 1, 8, 8, 64, 9, FAKE, None, FAKE, 0, None) == 1
    assert lib.ca_route(FAKE, FAKE, 1, 1, 8, 8, 64, 0, FAKE, None, FAKE, 0, None) == 1
    assert lib.ca_route(FAKE, FAKE, 1, 1, 8, 9000, 64, 4, FAKE, None, FAKE, 0, None) == 2
    assert lib.ca_route(FAKE, FAKE, 1, 1, 8, 8, 64, 4, FAKE, None, FAKE, 16, None) == 3
    assert lib.ca_dense(FAKE, FAKE, None, 0, 1, 1, 128, 64, 0.0, FAKE, None, FAKE, 0, None) == 1
    assert lib.ca_dense(FAKE, FAKE, FAKE, 0, 1, 1, 128, 80, 0.0, FAKE, None, FAKE, 0, None) == 2
    assert lib.ca_dense(FAKE, FAKE, FAKE, 0, 1, 1, 128, 64, 0.0, FAKE, None, FAKE, 8, None) == 3


def test_route_noalloc_rejects_bad_arguments(lib):
    # cent_q, cent_k, B, H, n_qc, n_kc, D, topk, blocks, stream
    nr = lib.ca_route_noalloc
    assert nr(FAKE, FAKE, 1, 1, 8, 8, 64, 4, None, None) == 1
    assert nr(FAKE, FAKE, 1, 1, 8, 8, 64, 9, FAKE, None) == 1
    assert nr(FAKE, FAKE, 1, 1, 8, 8, 96, 4, FAKE, None) == 2
    # beyond the 8388608-score scratch: refused on the host, before any HIP call
    assert nr(FAKE, FAKE, 1, 9, 1024, 1024, 64, 4, FAKE, None) == 2
    assert b"scratch" in lib.ca_last_error()
    assert nr(FAKE, FAKE, 2, 4, 1024, 1025, 64, 4, FAKE, None) == 2


def test_adaptive_route_and_ragged_attend_reject_bad_arguments(lib):
    ra = lib.ca_route_adaptive
    # cent_q, cent_k, counts, B, H, n_qc, n_kc, D, scale, recall, min_count, blocks, nsel, scores, ws
    assert ra(FAKE, FAKE, None, 1, 1, 8, 8, 64, 0.0, 0.9, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == 1
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, 0.0, 1.5, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == 1
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, 0.0, -0.1, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == 1
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, 0.0, 0.9, 0, FAKE, FAKE, None, FAKE, 1 << 20, None) == 1
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, -1.0, 0.9, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == 1
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 96, 0.0, 0.9, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == 2
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 9000, 64, 0.0, 0.9, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == 2
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, 0.0, 0.9, 16, FAKE, None, None, FAKE, 1 << 20, None) == 1
    assert ra(FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, 0.0, 0.9, 16, FAKE, FAKE, None, FAKE, 16, None) == 3
    av = lib.ca_attend_var
    # Q, K, V, dt, B, H, N, D, perm_q, perm_k, c, blocks, nsel, max_sel, comp, scale, O, lse, ws
    assert av(FAKE, FAKE, FAKE, 0, 1, 1, 1024, 64, FAKE, FAKE, 64, FAKE, None, 4, 1, 0.0, FAKE, None,
              FAKE, 1 << 30, None) == 1
    assert av(FAKE, FAKE, FAKE, 0, 1, 1, 1024, 64, FAKE, FAKE, 64, FAKE, FAKE, 17, 1, 0.0, FAKE,
              None, FAKE, 1 << 30, None) == 1
    assert av(FAKE, FAKE, FAKE, 0, 1, 1, 1024, 64, FAKE, FAKE, 64, FAKE, FAKE, 0, 1, 0.0, FAKE,
              None, FAKE, 1 << 30, None) == 1
    assert av(FAKE, FAKE, FAKE, 0, 1, 1, 1024, 64, FAKE, FAKE, 64, FAKE, FAKE, 4, 1, 0.0, FAKE,
              None, FAKE, 10, None) == 3


def test_peak_probe_rejects_bad_arguments(lib):
    assert lib.ca_peak_probe(2, 1, 1, FAKE, None) == 1
    assert lib.ca_peak_probe(0, 0, 1, FAKE, None) == 1
    assert lib.ca_peak_probe(1, 1, 0, FAKE, None) == 1
    assert lib.ca_peak_probe(0, 1, 1, None, None) == 1


def test_fp8_dtype_and_quantize_reject_bad_arguments(lib):
    # CA_BF16_FP8 (2) is for attention only: ca_cluster rejects it, ca_dense
    # and ca_attend take it (then fail here on the workspace, nothing launched)
    assert _cluster(lib, dt=2) == 1
    assert b"attention only" in lib.ca_last_error()
    assert lib.ca_dense(FAKE, FAKE, FAKE, 2, 1, 1, 128, 64, 0.0, FAKE, None, FAKE, 8, None) == 3
    # CA_BF16_FP8_PV (3): attention only, query clusters of 128 or 256
    assert lib.ca_dense(FAKE, FAKE, FAKE, 3, 1, 1, 128, 64, 0.0, FAKE, None, FAKE, 8, None) == 3
    assert lib.ca_dense(FAKE, FAKE, FAKE, 4, 1, 1, 128, 64, 0.0, FAKE, None, FAKE, 8, None) == 1
    assert _cluster(lib, dt=3) == 1
    assert _attend(lib, dt=3, c=64) == 2
    assert b"CA_BF16_FP8_PV" in lib.ca_last_error()
    assert _attend(lib, dt=3, c=128, topk=2, ws_bytes=10) == 3
    assert _attend(lib, dt=2, ws_bytes=10) == 3
    q = lib.ca_quantize_e4m3
    # X, dt, rows, D, group, codes, scales, stream
    assert q(None, 0, 4, 64, 1, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 4, 64, 1, None, FAKE, None) == 1
    assert q(FAKE, 0, 4, 64, 1, FAKE, None, None) == 1
    assert q(FAKE, 2, 4, 64, 1, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 0, 64, 1, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 4, 0, 1, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 4, 64, 0, FAKE, FAKE, None) == 1
    assert q(FAKE, 1, 1 << 25, 64, 1, FAKE, FAKE, None) == 1


def test_kv_heads_rejected_unless_dividing_h(lib):
    import free_clustered_block_amd as ca
    opts = ca._Opts(1, 1, 8, 1, 0, None, None, None, 0, None, 0, 3)
    assert _cluster(lib, H=4, opts=ctypes.byref(opts)) == 1
    assert b"kv_heads" in lib.ca_last_error()
    opts = ca._Opts(1, 1, 8, 1, 0, None, None, None, 0, None, 0, 8)
    assert _cluster(lib, H=4, opts=ctypes.byref(opts)) == 1
    opts = ca._Opts(1, 1, 8, 1, 0, None, None, None, 0, None, 0, 2, 2)
    assert _cluster(lib, H=4, opts=ctypes.byref(opts)) == 1
    assert b"kv_share" in lib.ca_last_error()
    ex = lib.ca_attend_ex
    # Q, K, V, dt, B, H, kv_heads, kv_shared, N, D, perm_q, perm_k, c_q, c_k, blocks, nsel,
    # max_sel, comp, scale, O, lse, ws, ws_bytes, stream
    assert ex(FAKE, FAKE, FAKE, 0, 1, 4, 3, 0, 1024, 64, FAKE, FAKE, 64, 64, FAKE, None, 4, 1, 0.0,
              FAKE, None, FAKE, 1 << 30, None) == 1
    assert b"kv_heads" in lib.ca_last_error()
    assert ex(FAKE, FAKE, FAKE, 0, 1, 4, 2, 2, 1024, 64, FAKE, FAKE, 64, 64, FAKE, None, 4, 1, 0.0,
              FAKE, None, FAKE, 1 << 30, None) == 1
    assert b"kv_shared" in lib.ca_last_error()
    assert ex(FAKE, FAKE, FAKE, 0, 1, 4, 2, 1, 1024, 64, FAKE, FAKE, 64, 64, FAKE, None, 4, 1, 0.0,
              FAKE, None, FAKE, 10, None) == 3


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """The product path has no fallback: without libca.so every call raises."""
    import free_clustered_block_amd as ca
    monkeypatch.setattr(ca, "LIB_PATH", str(tmp_path / "missing" / "libca.so"))
    monkeypatch.setattr(ca, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        ca.load()
    with pytest.raises(RuntimeError, match="not built"):
        ca.workspace_size(ca.OP_ATTEND, 1, 1, 1024, 64, 64)


def test_product_path_does_not_import_the_oracle():
    """Only tests, the smoke check and the bench's CPU leg may use the oracle."""
    import pathlib
    pkg = pathlib.Path(ROOT) / "free_clustered_block_amd"
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.h")):
        text = f.read_text()
        assert "oracle" not in text, f


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message and
    touches no device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_calls_from_several_threads(lib):
    """The host side keeps no shared state on these paths: workspace sizing
    and argument validation from eight threads at once give each thread its
    own results and its own ca_last_error string."""
    import threading
    import free_clustered_block_amd as ca
    want_ws = ca.workspace_size(ca.OP_ATTEND, 1, 8, 65536, 64, 128, 64)
    errors = []

    def work(k):
        try:
            for i in range(200):
                assert ca.workspace_size(ca.OP_ATTEND, 1, 8, 65536, 64, 128, 64) == want_ws
                if (i + k) % 2:
                    assert _attend(lib, D=32) == 2
                    assert b"D must be" in lib.ca_last_error()
                else:
                    assert _cluster(lib, c=100) == 2
                    assert b"cluster_size" in lib.ca_last_error()
        except AssertionError as e:      # pragma: no cover - reported below
            errors.append((k, e))

    ts = [threading.Thread(target=work, args=(k,)) for k in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
