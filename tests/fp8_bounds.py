"""Error bound of FP8 attention weights (test logic, no method arithmetic of
the library): with the weights of a row taken as p = 2^(x - m_ref + 6)
rounded to E4M3 (x the score in log2 units, m_ref a reference with
m - 2 <= m_ref <= m, m the row max), the output of P.V over the rounded
weights, normalised by their sum, differs from the exact softmax output o
per dim by at most

    1.1 * 2^-4 * sum_i w_i |v_i - o|  +  2^-16 * sum_{x_i - m < -12} |v_i - o|

to first order: a weight in E4M3's normal range (p >= 2^-6, which holds for
every key with x_i - m >= -12) carries a relative error <= 2^-4 (half the
spacing of 3 mantissa bits); a smaller one an absolute error <= 2^-10 (half
the subnormal step), i.e. <= 2^-16 of the weight sum (>= 2^6, the row max's
weight); the normalisation turns the weight errors e_i into
sum_i e_i (v_i - o) / sum p; the factor 1.1 covers the second-order terms.
"""
import numpy as np


def fp8_pv_bound(x_log2, w, v, o):
    """x_log2 [n]: scores of the row's active keys in log2 units; w [n]: the
    exact softmax weights; v [n, d]: the values; o [d]: the exact output.
    Returns the per-dim bound [d]."""
    dev = np.abs(np.asarray(v, dtype=np.float64) - np.asarray(o, dtype=np.float64)[None, :])
    tiny = (x_log2 - x_log2.max()) < -12
    return 1.1 * 2.0 ** -4 * (np.asarray(w) @ dev) + 2.0 ** -16 * dev[tiny].sum(axis=0)
