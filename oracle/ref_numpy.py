"""Dense fp64 numpy restatement of the masks, permutation, attention and
profiling, for tiny shapes.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Written independently of svg_oracle.c so that the two cross-check each other:
masks are built by broadcasting the definitions over index grids instead of a
per-pair predicate, and softmax is a whole-matrix operation.

Definitions (rebuttal to "Weakness 1" on the Sparse Video-Gen page): token
x = i*F + j; spatial |floor(x1/F) - floor(x2/F)| < a1; temporal
|(x1 mod F) - (x2 mod F)| < a2.  The text prefix [0, T), window, stripe and
skip modes follow the same readings as the C oracle.
"""
import numpy as np

SPATIAL, TEMPORAL, FULL, SKIP, WINDOW, STRIPE = range(6)


def dense_mask(N, F, T, mode, a1=1, a2=1, window=1, stripe=1):
    L = T + N * F
    x = np.arange(L)
    x1, x2 = x[:, None], x[None, :]
    text = (x1 < T) | (x2 < T)
    u1, u2 = x1 - T, x2 - T
    if mode == SPATIAL:
        vid = np.abs(np.floor_divide(u1, F) - np.floor_divide(u2, F)) < a1
    elif mode == TEMPORAL:
        vid = np.abs(np.mod(u1, F) - np.mod(u2, F)) < a2
    elif mode == FULL:
        vid = np.ones((L, L), dtype=bool)
    elif mode == WINDOW:
        vid = np.abs(u1 - u2) < window
    elif mode == STRIPE:
        vid = np.broadcast_to(u2 < stripe, (L, L))
    elif mode == SKIP:
        return np.zeros((L, L), dtype=bool)
    else:
        raise ValueError(mode)
    return text | vid


def permutation(N, F, T):
    """pi[x]: token-major position of natural token x (text rows fixed)."""
    L = T + N * F
    pi = np.arange(L)
    i, j = np.divmod(np.arange(N * F), F)
    pi[T:] = T + j * N + i
    return pi


def attention(q, k, v, mask, scale):
    """softmax(q k^T * scale, masked) v in fp64; rows with no key -> 0."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    p = np.where(mask, np.exp(s - m), 0.0)
    l = p.sum(axis=1, keepdims=True)
    l = np.where(l == 0, 1.0, l)
    return (p / l) @ v, p / l


def profile(q, k, v, N, F, T, a1, a2, scale, rows, fallback=0.05):
    o_f, _ = attention(q, k, v, dense_mask(N, F, T, FULL), scale)
    o_s, _ = attention(q, k, v, dense_mask(N, F, T, SPATIAL, a1=a1), scale)
    o_t, _ = attention(q, k, v, dense_mask(N, F, T, TEMPORAL, a2=a2), scale)
    o_f, o_s, o_t = o_f[rows], o_s[rows], o_t[rows]
    den = np.sum(o_f * o_f)
    rel_s = np.sum((o_s - o_f) ** 2) / den
    rel_t = np.sum((o_t - o_f) ** 2) / den
    if min(rel_s, rel_t) >= fallback:
        label = FULL
    else:
        label = SPATIAL if rel_s <= rel_t else TEMPORAL
    return label, np.array([rel_s, rel_t, den / o_f.size])
