#!/usr/bin/env python3
"""Benchmark of the ClusterAttention forward hot path on one MI355X (gfx950).

One step is one pass of the whole path over one batch of synthetic input:
ca_cluster (metrics, recursive PDDP splitting of queries and keys, centroids)
-> ca_route (centroid scores, top-k) -> ca_attend (key/value tiles and
centroids, block-sparse attention with striped mean-compensation).

Default workload: the Wan-2.1-14B-like video self-attention shape, 40 heads,
N = 32760 tokens (21x30x52 latent grid), head_dim 128, bf16, cluster size 128,
top 1/8 of key clusters (32), compensation on. Inputs are generated on the host
(seeded), uploaded once, and resident in HBM before the timed region.

Prints one JSON line:
  value      dense-equivalent effective TFLOP/s = 4 d N^2 H / step time
  roofline   the block-sparse attention kernel against the bf16 MFMA peak,
             counting 4 d FLOP per performed token or centroid interaction,
             timed with HIP events recorded around that kernel alone
  cpu_baseline  the CPU oracle on a bounded sample of heads of the same input
The headline (value, ms_per_step) is the median of the K timed steps, each
run after a 512 MiB write that flushes the L2 caches and the 256 MB MALL
(cold), timed by HIP events around the step; the same K steps run back to back
(warm) are reported beside it with per-stage times. Also reported: the
measured HBM copy and bf16 GEMM rates of the box (a 1 GiB torch copy, which
also serves as the plain-copy calibration of the HBM byte counters, and an
8192^3 torch.matmul), and the same forward on the tabular workloads
(8 x 65536 and 8 x 262144 tokens, d 64) under "other_workloads".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ClusterAttention fwd latency, eff. TFLOP/s & speedup vs dense at N=32k, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
# FP8 Q.K^T with bf16 P.V: half the FLOPs at each rate, so the bound on the
# whole count is 4 / (2 / 5000 + 2 / 2500) TFLOP/s
PEAK_FP8QK_TFLOPS = 4.0 / (2.0 / PEAK_FP8_TFLOPS + 2.0 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0
# HBM bytes per attention launch from rocprofv3 FETCH_SIZE + WRITE_SIZE runs,
# scaled by the same counters on a plain copy; valid only for the kernel
# sources whose digest the file records.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_video_32760_traffic.txt")
TRAFFIC_FILE_FP8 = os.path.join(ROOT, "profiles", "attn_fwd_fp8_video_32760_traffic.txt")
ATTN_SOURCES = ["attn.hip", "fp8.h", "mfma.h", "common.h", "kernels.h"]


def attn_source_digest() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "free_clustered_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str, topk: int, fp8: bool = False):
    """HBM bytes per attention launch recorded for this workload and these
    kernel sources, or None."""
    try:
        kv = {}
        with open(TRAFFIC_FILE_FP8 if fp8 else TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith(("#", " ", "|")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if (kv.get("workload") == workload and int(kv.get("topk", -1)) == topk
                and kv.get("sources_sha256") == attn_source_digest()):
            return float(kv["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video_32760")
    ap.add_argument("--topk", type=int, default=0, help="override top-k")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-sdpa", action="store_true",
                    help="skip the torch scaled_dot_product_attention (flash backend) reference")
    ap.add_argument("--cpu-heads", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--others", default="tabular_64k,tabular_256k",
                    help="further workloads timed in the same run (comma-separated; '' for none)")
    ap.add_argument("--other-steps", type=int, default=5)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the copy and GEMM rate measurements")
    ap.add_argument("--split-mode", choices=["power", "diag"], default="power",
                    help="basic (power iteration) or diagonalized recursive splitting")
    ap.add_argument("--cq", type=int, default=0,
                    help="query cluster size when it differs from the key cluster size")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--assign", choices=["topk", "adaptive"], default="topk",
                    help="top-k selection, or adaptive selection to a mass recall")
    ap.add_argument("--recall", type=float, default=0.9, help="mass recall of --assign adaptive")
    ap.add_argument("--min-count", type=int, default=16, help="minimum count of --assign adaptive")
    ap.add_argument("--fp8", action="store_true",
                    help="Q.K^T on FP8 (E4M3) operands in the attention and in the dense "
                         "baseline (dtype CA_BF16_FP8); P.V stays bf16")
    ap.add_argument("--fp8-pv", action="store_true",
                    help="Q.K^T and P.V on FP8 (E4M3) operands (dtype CA_BF16_FP8_PV), in the "
                         "attention and in the dense baseline")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="shared key/value heads (grouped- or multi-query attention): K and V "
                         "keep the workload's first KV heads; every query head clusters its "
                         "KV head's keys under its own metric")
    ap.add_argument("--kv-share", action="store_true",
                    help="with --kv-heads: one key clustering per KV head under the mean of its "
                         "query heads' metrics")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="quality/latency sweep over cluster size, selected fraction, SMC and "
                         "clustering (the 16k peaked and flat workloads); one JSON line per point")
    return ap.parse_args()


def gen_inputs(w):
    import synth
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        parts = list(ex.map(lambda h: synth.generate(w, heads=slice(h, h + 1)), range(w.H)))
    Q = np.concatenate([p[0] for p in parts], axis=1)
    K = np.concatenate([p[1] for p in parts], axis=1)
    V = np.concatenate([p[2] for p in parts], axis=1)
    return Q, K, V


def host_info():
    """CPU model and the BLAS numpy runs on (vendor, version, threads)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "arch": i.get("architecture")}
                break
    except Exception:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas": blas}


def oracle_small_case(synth):
    """The oracle on the whole 1024-token fp32 workload (1 head, d 64, c 64,
    top 4), with the BLAS threads as set and with one thread."""
    import oracle.clusterattn as o
    from threadpoolctl import threadpool_limits
    w = synth.WORKLOADS["small_gmm_1k"]
    Q, K, V = synth.generate(w)
    opts = o.ClusterOpts(seed=w.cluster_seed)
    out = {"workload": w.name}
    for label, limit in (("all_threads_s", None), ("one_thread_s", 1)):
        ts = []
        for _ in range(3):
            with threadpool_limits(limits=limit):
                t0 = time.perf_counter()
                o.forward(Q, K, V, w.c, w.topk, w.compensate, opts, w.dtype)
                ts.append(time.perf_counter() - t0)
        out[label] = round(float(np.median(ts)), 4)
    return out


def cpu_baseline(w, Q, K, V, topk, heads, split_mode="power", assign="topk", recall=0.9,
                 min_count=16, qk="exact", pv="exact"):
    """The oracle, untuned, on the first `heads` heads of the same input."""
    import oracle.clusterattn as o
    info = host_info()
    cores = int(info["blas"].get("threads") or 1)
    opts = o.ClusterOpts(seed=w.cluster_seed, split_mode=split_mode,
                         query_normalize=assign == "topk")
    t0 = time.perf_counter()
    if assign == "topk":
        o.forward(Q[:, :heads], K[:, :heads], V[:, :heads], w.c, topk, w.compensate, opts, w.dtype,
                  qk=qk, pv=pv)
    else:
        Qs, Ks, Vs = Q[:, :heads], K[:, :heads], V[:, :heads]
        pq, pk = o.cluster(Qs, Ks, w.c, opts, w.dtype)
        tau = 1.0 / math.sqrt(w.D)
        sel = [[None] * heads for _ in range(w.B)]
        for b in range(w.B):
            for h in range(heads):
                cq, _ = o.centroids(Qs[b, h], pq[b, h], w.c)
                ck, cnt = o.centroids(Ks[b, h], pk[b, h], w.c)
                sel[b][h] = o.route_adaptive(cq, ck, cnt, tau, recall, min_count)
        o.attend(Qs, Ks, Vs, pq, pk, w.c, sel, w.compensate, qk=qk, pv=pv)
    t = time.perf_counter() - t0
    flops = 4.0 * w.D * w.N * w.N * heads * w.B
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{heads} of {w.H} heads of the same workload, full N={w.N}; "
                  f"{t:.2f} s wall for cluster+route+attend in fp64 NumPy"
                  f"{' (FP8 Q.K^T operands)' if qk == 'e4m3' and pv != 'e4m3' else ''}"
                  f"{' (FP8 Q.K^T and P.V operands)' if pv == 'e4m3' else ''} "
                  f"(BLAS threads={cores}; PDDP and top-k loops single-threaded Python)",
        "seconds": t,
        **info,
    }


def measure_peaks(torch, dev):
    """Achievable rates of this machine: a plain 1 GiB bf16 copy (read + write
    bytes over time; also the calibration kernel for the HBM byte counters)
    and a bf16 8192^3 GEMM through torch.matmul."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for a_ev, b_ev in ev:
        a_ev.record()
        dst.copy_(src)
        b_ev.record()
    torch.cuda.synchronize()
    copy_ms = float(np.median([a_ev.elapsed_time(b_ev) for a_ev, b_ev in ev]))
    del src, dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    b = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    torch.matmul(a, b)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for a_ev, b_ev in ev:
        a_ev.record()
        torch.matmul(a, b)
        b_ev.record()
    torch.cuda.synchronize()
    gemm_ms = float(np.median([a_ev.elapsed_time(b_ev) for a_ev, b_ev in ev]))
    del a, b
    # matrix-core and LDS probes of the library: 2 workgroups of 4 waves per CU
    import free_clustered_block_amd as ca
    blocks, iters = 512, 20000
    out = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    rates = {}
    for kind, name in ((0, "mfma"), (1, "lds")):
        ca.peak_probe(kind, blocks, 100, out)
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record()
        ca.peak_probe(kind, blocks, iters, out)
        b_ev.record()
        torch.cuda.synchronize()
        rates[name] = a_ev.elapsed_time(b_ev) * 1e-3
    mfma_tf = blocks * 4 * 4 * iters * 32768.0 / rates["mfma"] / 1e12
    lds_tbs = blocks * 4 * 8 * iters * 1024.0 / rates["lds"] / 1e12
    return {"hbm_copy_GBs": round(2.0 * n * 2 / (copy_ms * 1e-3) / 1e9, 1),
            "copy_bytes": 2 * n * 2,
            "bf16_gemm_TFLOPs": round(2.0 * m ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "mfma_loop_TFLOPs": round(mfma_tf, 1),
            "lds_read_TBs": round(lds_tbs, 2)}


def sweep(args, torch, synth, ca):
    """Error against dense attention and latency over cluster size c in {64, 128, 256},
    selected fraction k/n_c in {1/4, 1/8, 1/16}, SMC off/on, for the learned
    (PDDP) clusters and for seeded random clusters of the same sizes; then
    adaptive selection at mass recalls {0.6, 0.8, 0.9, 0.95, 0.99} (minimum
    count 16), SMC off/on. With --fp8 the attention takes FP8 Q.K^T operands,
    the latency is compared with FP8 dense attention and the error with bf16
    dense attention."""
    dev = torch.device("cuda:0")

    def timed(fn, reps=3):
        out, ts = None, []
        for _ in range(reps):
            a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_ev.record()
            out = fn()
            b_ev.record()
            torch.cuda.synchronize()
            ts.append(a_ev.elapsed_time(b_ev))
        return out, float(np.median(ts))

    for regime in ("peaked", "flat"):
        w = synth.WORKLOADS[f"sweep_16k_{regime}"]
        Qn, Kn, Vn = gen_inputs(w)
        Q, K, V = (torch.from_numpy(x).to(torch.bfloat16).to(dev).contiguous() for x in (Qn, Kn, Vn))
        B, H, N, D = Q.shape
        Od, dense_ms = timed(lambda: ca.dense(Q, K, V, fp8=args.fp8))
        if args.fp8:
            Od = ca.dense(Q, K, V)   # the error reference stays bf16 dense attention
        Odf = Od.float()
        nd = torch.linalg.vector_norm(Odf).item()
        for c in (64, 128, 256):
            n_c = N // c
            # random clusters of the same sizes: seeded shuffles, centroids by mean
            pq = torch.from_numpy(synth.random_perm(w.control_seed, B, H, N)).to(dev)
            pk = torch.from_numpy(synth.random_perm(w.control_seed + 1, B, H, N)).to(dev)

            def cent(X, perm):
                Xg = torch.gather(X.float(), 2, perm.long()[..., None].expand(-1, -1, -1, D))
                return Xg.view(B, H, n_c, c, D).mean(3).contiguous()
            rq, rk = cent(Q, pq), cent(K, pk)
            for f in (4, 8, 16):
                k = n_c // f
                for smc in (False, True):
                    for kind in ("pddp", "random"):
                        def run():
                            if kind == "pddp":
                                cr = ca.cluster(Q, K, c, seed=w.cluster_seed)
                                bl = ca.route(cr.cent_q, cr.cent_k, k)
                                return ca.attend(Q, K, V, cr.perm_q, cr.perm_k, c, bl, compensate=smc,
                                                 fp8=args.fp8)
                            bl = ca.route(rq, rk, k)
                            return ca.attend(Q, K, V, pq, pk, c, bl, compensate=smc, fp8=args.fp8)
                        O, ms = timed(run)
                        Of = O.float()
                        rel = torch.linalg.vector_norm(Of - Odf).item() / nd
                        cos = torch.nn.functional.cosine_similarity(Of, Odf, dim=-1).mean().item()
                        print(json.dumps({"sweep": w.name, "fp8": args.fp8, "clusters": kind, "c": c, "k": k,
                                          "fraction": f"1/{f}", "smc": smc,
                                          "rel_err_vs_dense": round(rel, 5),
                                          "cos_vs_dense": round(cos, 5), "ms": round(ms, 4),
                                          "dense_ms": round(dense_ms, 4),
                                          "speedup_vs_dense": round(dense_ms / ms, 3)}), flush=True)
            # adaptive selection to a mass recall (queries clustered unnormalised)
            for recall in (0.6, 0.8, 0.9, 0.95, 0.99):
                for smc in (False, True):
                    sel = {}

                    def run_ada():
                        cr = ca.cluster(Q, K, c, seed=w.cluster_seed, query_normalize=False)
                        bl, ns = ca.route_adaptive(cr.cent_q, cr.cent_k, cr.counts, recall,
                                                   min_count=16)
                        sel["n"] = ns
                        return ca.attend(Q, K, V, cr.perm_q, cr.perm_k, c, bl, compensate=smc,
                                         nsel=ns, fp8=args.fp8)
                    O, ms = timed(run_ada)
                    Of = O.float()
                    rel = torch.linalg.vector_norm(Of - Odf).item() / nd
                    cos = torch.nn.functional.cosine_similarity(Of, Odf, dim=-1).mean().item()
                    frac = sel["n"].float().mean().item() / n_c
                    print(json.dumps({"sweep": w.name, "fp8": args.fp8, "clusters": "pddp", "assign": "adaptive",
                                      "c": c, "recall": recall, "selected_fraction": round(frac, 4),
                                      "smc": smc, "rel_err_vs_dense": round(rel, 5),
                                      "cos_vs_dense": round(cos, 5), "ms": round(ms, 4),
                                      "dense_ms": round(dense_ms, 4),
                                      "speedup_vs_dense": round(dense_ms / ms, 3)}), flush=True)


def run_workload(args, wname, torch, synth, ca, dev, steps, warmup, full=True):
    """Times the forward on one workload; returns the result dict (the JSON
    line's fields). full=False skips the torch SDPA reference, the peaks and
    the CPU baseline (the extra workloads of one run)."""
    w = synth.WORKLOADS[wname]
    topk = (args.topk or w.topk) if full else w.topk
    t_gen = time.perf_counter()
    Qn, Kn, Vn = gen_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Q = torch.from_numpy(Qn).to(tdt).to(dev).contiguous()
    kvh = (args.kv_heads or w.H) if full else w.H
    if w.H % kvh != 0:
        print("--kv-heads must divide the workload's head count", file=sys.stderr)
        sys.exit(2)
    if kvh != w.H:
        # the first kvh heads' keys and values, shared by H / kvh query heads each
        Kn = np.ascontiguousarray(Kn[:, :kvh])
        Vn = np.ascontiguousarray(Vn[:, :kvh])
    K = torch.from_numpy(Kn).to(tdt).to(dev).contiguous()
    V = torch.from_numpy(Vn).to(tdt).to(dev).contiguous()
    if args.verbose:
        print(f"{wname}: inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr,
              flush=True)
    B, H, N, D = Q.shape
    c = w.c                                  # key cluster size
    cq = (args.cq or c) if full else c       # query cluster size
    split_mode = args.split_mode if full else "power"
    adaptive = full and args.assign == "adaptive"
    fp8 = ("qkpv" if args.fp8_pv else args.fp8) if full else False
    kv_share = full and args.kv_share
    op_c = ca.OP_CLUSTER_DIAG if split_mode == "diag" else ca.OP_CLUSTER
    ws_c = torch.empty(ca.workspace_size(op_c, B, H, N, D, min(c, cq)), dtype=torch.uint8,
                       device=dev)
    n_c = -(-N // c)
    n_qc = -(-N // cq)
    ws_r = torch.empty(max(1, ca.workspace_size(ca.OP_ROUTE, B, H, n_qc, D, n_c, topk)),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty(ca.workspace_size(ca.OP_ATTEND, B, H, N, D, c, topk), dtype=torch.uint8,
                       device=dev)

    def step(evs=None, kev=None):
        if evs:
            evs[0].record()
        cr = ca.cluster(Q, K, cq, seed=w.cluster_seed, split_mode=split_mode,
                        query_normalize=not adaptive, cluster_size_k=c if cq != c else 0,
                        kv_share=kv_share, workspace=ws_c)
        if evs:
            evs[1].record()
        if adaptive:
            blocks, nsel = ca.route_adaptive(cr.cent_q, cr.cent_k, cr.counts, args.recall,
                                             min_count=args.min_count, workspace=ws_r)
        else:
            blocks, nsel = ca.route(cr.cent_q, cr.cent_k, topk, workspace=ws_r), None
        if evs:
            evs[2].record()
            if kev is not None:
                ca.profile_events(kev[0].handle, kev[1].handle)
        O = ca.attend(Q, K, V, cr.perm_q, cr.perm_k, cq, blocks, compensate=w.compensate,
                      nsel=nsel, c_k=c, fp8=fp8, kv_shared=kv_share, workspace=ws_a)
        if evs:
            if kev is not None:
                ca.profile_events(None, None)
            evs[3].record()
        return O, cr, (blocks, nsel)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # headline: K steps, each after a 512 MiB write that flushes the L2 caches
    # and the MALL; HIP events around the step alone
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)]
    torch.cuda.synchronize()
    tc = time.perf_counter()
    for i in range(steps):
        flush.fill_(i & 0xFF)
        cold[i][0].record()
        step()
        cold[i][1].record()
    torch.cuda.synchronize()
    cold_wall = (time.perf_counter() - tc) / steps
    del flush
    cold_ms = np.array([a.elapsed_time(b) for a, b in cold])

    # warm: the same K steps back to back, with per-stage events and the
    # attention kernel's own events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    kevs = [(ca.HipEvent(), ca.HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        O, cr, blocks = step(evs[i], kevs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    if args.verbose:
        print(f"{wname}: cold median {np.median(cold_ms):.3f} ms, warm {wall * 1e3:.3f} ms/step",
              file=sys.stderr, flush=True)
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    st_cluster = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    st_route = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    st_attend = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    t_attn_kernel = np.mean([a.elapsed_ms(b) for a, b in kevs])
    gpu_step = np.mean([e[0].elapsed_time(e[3]) for e in evs])

    # performed interactions of the attention kernel (valid keys and centroids)
    blocks, nsel = blocks
    bl = blocks.cpu().numpy().astype(np.int64)
    sizes = np.full(n_c, c, np.int64)
    sizes[-1] = N - (n_c - 1) * c
    if nsel is None:
        ns = np.full(bl.shape[:3], topk, np.int64)
    else:
        ns = nsel.cpu().numpy().astype(np.int64)
    take = np.arange(bl.shape[-1])[None, None, None, :] < ns[..., None]
    sel_sizes = np.where(take, sizes[np.clip(bl, 0, n_c - 1)], 0).sum(-1)
    qsizes = np.full(n_qc, cq, np.int64)
    qsizes[-1] = N - (n_qc - 1) * cq
    tok_inter = float(np.sum(qsizes[None, None, :] * sel_sizes))
    cen_inter = float(np.sum(qsizes[None, None, :] * (n_c - ns))) if w.compensate else 0.0
    mean_sel = float(ns.mean())
    flops_attn = 4.0 * D * (tok_inter + cen_inter)
    achieved = flops_attn / (t_attn_kernel * 1e-3) / 1e12

    # the same step captured once in a HIP graph (fixed shapes) and replayed
    graph_ms = None
    if full and args.graph:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            step()
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg) / steps * 1e3
        del graph

    # clustering + routing against the HBM roofline. Algorithmic bytes: per
    # tree actually built, per split level and token, the row read for the
    # projection plus the index read and write (2 D e + 8 B, e = element
    # size); plus the compulsory metric pass (every query row and every key
    # row of the key/value heads) and centroid pass (query rows per head, key
    # and value rows per key tree).
    esz = 2 if w.dtype == "bf16" else 4
    row = N * D * esz
    key_trees = B * (H // (H // kvh) if kv_share else H)
    q_trees = B * H
    clu_bytes = float(q_trees * ca.tree_levels(N, cq) * N * (D * esz + 8)
                      + key_trees * ca.tree_levels(N, c) * N * (D * esz + 8)
                      + (q_trees + B * kvh) * row + (q_trees + 2 * key_trees) * row)
    clu_ms = float(st_cluster + st_route)
    clu_gbs = clu_bytes / (clu_ms * 1e-3) / 1e9

    traffic = (recorded_traffic(w.name, topk, bool(fp8)) if B * H == w.B * w.H and not adaptive
               and split_mode == "power" and cq == c and kvh == w.H and fp8 != "qkpv" else None)
    peak = (PEAK_FP8_TFLOPS if fp8 == "qkpv" else PEAK_FP8QK_TFLOPS if fp8 else PEAK_BF16_TFLOPS)
    dense_eq = 4.0 * D * N * N * B * H
    head_ms = float(np.median(cold_ms))
    result = {
        "metric": METRIC,
        "value": round(dense_eq / (head_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s (dense-equivalent, 4 d N^2 H per step)",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(head_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 (Q.K^T and P.V)" if fp8 == "qkpv" else "fp8e4m3 (Q.K^T) + bf16 (P.V)" if fp8
                  else "bf16" if w.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "N": N, "head_dim": D,
                   "cluster_size": c, "topk": topk, "compensate": w.compensate,
                   "split_mode": split_mode, "assign": "adaptive" if adaptive else "topk",
                   **({"qk_operands": "fp8 e4m3, per-token query / per-64-key scales"}
                      if fp8 else {}),
                   **({"pv_operands": "fp8 e4m3, values with a power-of-two scale per "
                                      "dimension and 32 keys, weights unscaled"}
                      if fp8 == "qkpv" else {}),
                   **({"query_cluster_size": cq} if cq != c else {}),
                   **({"kv_heads": kvh, "kv_share": bool(kv_share)} if kvh != w.H else {}),
                   **({"recall": args.recall, "min_count": args.min_count,
                       "mean_selected": round(mean_sel, 2)} if adaptive else {})},
        "timing": ("value and ms_per_step: median of the K timed steps, each after a 512 MiB "
                   "cache flush (cold), HIP events around the step; warm: the same K steps "
                   "back to back"),
        "cold": {"ms_median": round(head_ms, 4), "ms_p10": round(float(np.percentile(cold_ms, 10)), 4),
                 "ms_p90": round(float(np.percentile(cold_ms, 90)), 4),
                 "wall_ms_per_step_with_flush": round(cold_wall * 1e3, 4)},
        "warm": {"ms_per_step": round(wall * 1e3, 4),
                 "value": round(dense_eq / wall / 1e12, 3)},
        "stage_ms": {"cluster": round(float(st_cluster), 4), "route": round(float(st_route), 4),
                     "attend": round(float(st_attend), 4),
                     "attend_kernel": round(float(t_attn_kernel), 4),
                     "gpu_step_events": round(float(gpu_step), 4),
                     "step_median": round(float(np.median(step_ms)), 4),
                     "step_p10": round(float(np.percentile(step_ms, 10)), 4),
                     "step_p90": round(float(np.percentile(step_ms, 90)), 4),
                     "graph_replay": round(graph_ms, 4) if graph_ms is not None else None},
        "roofline": {
            "kernel": ("attn_fwd2 (pipelined block-sparse attention + SMC)"
                       if not fp8 and w.dtype == "bf16" and cq in (128, 256)
                       else "attn_fwd (block-sparse attention + SMC)"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(peak, 1),
            **({"peak_note": "half the FLOPs (Q.K^T) at the fp8 5.0 PFLOP/s peak, half "
                             "(P.V) at the bf16 2.5 PFLOP/s peak"} if fp8 is True else {}),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "flops_per_launch": flops_attn,
        },
        "cluster_route_hbm": {
            "bytes": clu_bytes, "ms": round(clu_ms, 4), "achieved": round(clu_gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(clu_gbs / PEAK_HBM_GBS, 4),
        },
    }

    if not args.no_dense:
        ws_d = torch.empty(ca.workspace_size(ca.OP_DENSE, B, H, N, D), dtype=torch.uint8, device=dev)

        # the dense baseline takes the key/value heads repeated per query head
        Kd = K.repeat_interleave(w.H // kvh, dim=1).contiguous() if kvh != w.H else K
        Vd = V.repeat_interleave(w.H // kvh, dim=1).contiguous() if kvh != w.H else V

        def time_dense(use_fp8):
            Od = ca.dense(Q, Kd, Vd, fp8=use_fp8, workspace=ws_d)
            torch.cuda.synchronize()
            de = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.dense_steps)]
            for a, b in de:
                a.record()
                Od = ca.dense(Q, Kd, Vd, fp8=use_fp8, workspace=ws_d)
                b.record()
            torch.cuda.synchronize()
            return Od, float(np.mean([a.elapsed_time(b) for a, b in de]))

        def cosine(x, y):
            return torch.nn.functional.cosine_similarity(x.float(), y.float(), dim=-1).mean().item()

        # the dense baseline in the path's own precision ("given equal
        # quantization"); with --fp8 the bf16 dense output is the reference of
        # both cosines
        Od, dense_ms = time_dense(fp8)
        result["dense_ms"] = round(dense_ms, 4)
        result["speedup_vs_dense"] = round(dense_ms / head_ms, 3)
        result["speedup_vs_dense_warm"] = round(dense_ms / (wall * 1e3), 3)
        result["dense_tflops"] = round(dense_eq / (dense_ms * 1e-3) / 1e12, 2)
        if fp8:
            Ob, dense_bf16_ms = time_dense(False)
            result["dense_bf16_ms"] = round(dense_bf16_ms, 4)
            result["cos_vs_dense"] = round(cosine(O, Ob), 5)
            result["cos_dense_fp8_vs_dense_bf16"] = round(cosine(Od, Ob), 5)
        else:
            result["cos_vs_dense"] = round(cosine(O, Od), 5)
        del Od

        # reference only: torch's fused dense attention (flash backend) on the
        # same bf16 inputs, 3 timed calls
        if full and not args.no_sdpa and w.dtype == "bf16":
            try:
                from torch.nn.attention import SDPBackend, sdpa_kernel
                with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                    torch.nn.functional.scaled_dot_product_attention(Q, Kd, Vd)
                    torch.cuda.synchronize()
                    se = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                          for _ in range(3)]
                    for a, b in se:
                        a.record()
                        torch.nn.functional.scaled_dot_product_attention(Q, Kd, Vd)
                        b.record()
                    torch.cuda.synchronize()
                sdpa_ms = float(np.median([a.elapsed_time(b) for a, b in se]))
                result["torch_sdpa_flash_ms"] = round(sdpa_ms, 4)
                result["speedup_vs_torch_sdpa"] = round(sdpa_ms / head_ms, 3)
            except Exception as e:   # not available on this build: reported as absent
                result["torch_sdpa_flash_ms"] = None
                if args.verbose:
                    print(f"torch SDPA reference unavailable: {e}", file=sys.stderr)

    if full and not args.no_peaks:
        result["measured_peaks"] = measure_peaks(torch, dev)

    if full and not args.no_cpu_baseline:
        heads = max(1, min(args.cpu_heads, H))
        if kvh != w.H:
            Kn = np.repeat(Kn, w.H // kvh, axis=1)
            Vn = np.repeat(Vn, w.H // kvh, axis=1)
        result["cpu_baseline"] = cpu_baseline(w, Qn, Kn, Vn, topk, heads, split_mode,
                                              "adaptive" if adaptive else "topk", args.recall,
                                              args.min_count, "e4m3" if fp8 else "exact",
                                              "e4m3" if fp8 == "qkpv" else "exact")
        result["cpu_baseline"]["small_fp32_case"] = oracle_small_case(synth)
    return result


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads would shard across GPUs with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import free_clustered_block_amd as ca

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ca.load()
    if args.sweep:
        sweep(args, torch, synth, ca)
        return
    dev = torch.device("cuda:0")
    result = run_workload(args, args.workload, torch, synth, ca, dev, args.steps, args.warmup)
    torch.cuda.empty_cache()
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        r = run_workload(args, name, torch, synth, ca, dev, args.other_steps, 2, full=False)
        torch.cuda.empty_cache()
        others[name] = {k: r[k] for k in ("config", "ms_per_step", "value", "warm", "stage_ms",
                                          "dense_ms", "speedup_vs_dense", "cos_vs_dense")
                        if k in r}
        others[name]["roofline_frac"] = r["roofline"]["frac"]
        others[name]["cluster_route_hbm_frac"] = r["cluster_route_hbm"]["frac"]
        if args.verbose:
            print(f"{name}: {others[name]['ms_per_step']} ms", file=sys.stderr, flush=True)
    if others:
        result["other_workloads"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
