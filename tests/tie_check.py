"""End-to-end clustering acceptance: agreement with the oracle's own tree, and
every disagreement at a median tie.

A token whose cluster differs between the GPU's tree and the oracle's fp64
tree must have left the oracle's path at a split where its oracle score sits
at the split threshold: at the first level where the two paths put it in
different nodes, |score - threshold| <= TIE_FRACTION x the interquartile range
of the oracle's scores in that node (the threshold is the midpoint of the
t-th and (t+1)-th smallest scores, t the node's left size). The tree layout
depends only on (N, c), so a node is identified by its position range in
both trees. Paper: "ClusterAttention: A training-free speedup of
bidirectional attention" (arXiv 2608.26965), v1 §3.2.1 and the later
revision §4.1.1 (values at the split are partitioned arbitrarily).
"""
import bisect

import numpy as np

import oracle.clusterattn as o

AGREEMENT_FLOOR = 0.999
TIE_FRACTION = 1e-3


def _node_at(levels_off, levels, level, pos):
    if level >= len(levels):
        return None
    offs = levels_off[level]
    k = bisect.bisect_right(offs, pos) - 1
    if k < 0:
        return None
    nd = levels[level][k]
    return nd if nd.off <= pos < nd.off + nd.n else None


def tie_distances(gpu_perm, oracle_perm, trace, N, c):
    """For each token whose leaf differs: (token, level of the split, its
    oracle score's distance to the threshold in units of the node's IQR)."""
    gpu_perm = np.asarray(gpu_perm, np.int64)
    oracle_perm = np.asarray(oracle_perm, np.int64)
    inv_g = np.empty(N, np.int64); inv_g[gpu_perm] = np.arange(N)
    inv_o = np.empty(N, np.int64); inv_o[oracle_perm] = np.arange(N)
    leaf_g = np.asarray(inv_g) // c
    leaf_o = np.asarray(inv_o) // c
    levels = o.tree_levels(N, c)
    offs = [[nd.off for nd in lv] for lv in levels]
    out = []
    for i in np.flatnonzero(leaf_g != leaf_o):
        lvl = 0
        while True:
            ng = _node_at(offs, levels, lvl + 1, inv_g[i])
            no = _node_at(offs, levels, lvl + 1, inv_o[i])
            if ng is None or no is None or ng.off != no.off:
                break
            lvl += 1
        parent = _node_at(offs, levels, lvl, inv_o[i])
        before = trace.perms[lvl]
        pos = int(np.flatnonzero(before == i)[0])
        sc = trace.scores[lvl]
        ns = np.sort(sc[parent.off:parent.off + parent.n])
        t = o.split_size(parent.n, c)
        thr = 0.5 * (ns[t - 1] + ns[t])
        iqr = float(np.subtract(*np.percentile(ns, [75, 25])))
        out.append((int(i), lvl, abs(float(sc[pos]) - thr) / max(iqr, 1e-300)))
    return out


def check_tree(gpu_perm, oracle_perm, trace, N, c, label=""):
    """Asserts the acceptance on one tree and returns (agreement, worst tie
    distance in IQR units or 0)."""
    ag = o.cluster_agreement(np.asarray(gpu_perm), np.asarray(oracle_perm), c)
    ties = tie_distances(gpu_perm, oracle_perm, trace, N, c)
    worst = max((d for _, _, d in ties), default=0.0)
    assert ag >= AGREEMENT_FLOOR, (label, ag)
    bad = [x for x in ties if x[2] > TIE_FRACTION]
    assert not bad, (label, "disagreements not at a median tie (token, level, distance/IQR)", bad[:8])
    return ag, worst
