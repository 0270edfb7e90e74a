"""Bound on the effect of rounding the attention weights to E4M3 in the FP8
P.V product, for comparing the kernel with the oracle (which keeps the
weights exact).

The kernel forms P_j = 2^(l_j - m) against its running maximum m (at most
2^8, since m trails the largest logit by at most 8 in log2 units), rounds
P_j to the nearest E4M3 value P^_j and accumulates sum P^_j v^_j; the
denominator sums the unrounded P_j, and a later rescaling by 2^(m - m')
multiplies both alike. So O^ - O = sum_j (P^_j - P_j) v^_j / sum_j P_j, with
|P^_j - P_j| <= e(P_j) = max(2^-4 P_j, min(P_j, 2^-10)) (half a spacing:
2^-4 relative in the normal range, 2^-10 among the subnormals, at most P_j
when it rounds to 0). The bound is evaluated with m at the largest logit:
scaling every P_j by c >= 1 can only shrink e(c P) / (c sum P).
"""
import numpy as np


def pv_rounding_bound(logits, vals):
    """logits [rows, terms] (natural log units), vals [terms, D] (the values
    the weights multiply): per output element the largest |O^ - O|."""
    logits = np.asarray(logits, np.float64)
    P = np.exp(logits - logits.max(axis=1, keepdims=True))
    e = np.maximum(2.0 ** -4 * P, np.minimum(P, 2.0 ** -10))
    return (e @ np.abs(np.asarray(vals, np.float64))) / P.sum(axis=1, keepdims=True)
