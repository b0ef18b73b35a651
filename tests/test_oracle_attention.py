"""Pins of the oracle's masked attention (CPU only).

Special cases that reduce to a library routine (torch's scaled-dot-product
attention on the CPU in float64 with a boolean mask), normalisation
invariants (rows of P sum to one, masked entries are exactly zero, constant
values pass through), the dense limit, and the permutation equivariance that
the layout transformation relies on.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import ref_numpy as R

MODES = [oracle.SPATIAL, oracle.TEMPORAL, oracle.FULL, oracle.WINDOW, oracle.STRIPE]


def rand_qkv(L, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((L, d)) * scale).astype(np.float32)
    k = (rng.standard_normal((L, d)) * scale).astype(np.float32)
    v = rng.standard_normal((L, d)).astype(np.float32)
    return q, k, v


def sdpa(q, k, v, mask, scale):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))[None, None]
    m = torch.from_numpy(np.asarray(mask, dtype=bool))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("N,F,T,d", [(3, 4, 0, 8), (4, 5, 2, 16), (2, 7, 3, 5), (5, 3, 0, 4)])
def test_attention_vs_sdpa(oracle_lib, N, F, T, d):
    g = oracle.geom(N, F, T, 2, 2, window=3, stripe=4)
    L = T + N * F
    q, k, v = rand_qkv(L, d, seed=N * 100 + F, scale=1.5)
    scale = 1.0 / np.sqrt(d)
    for mode in MODES:
        m = R.dense_mask(N, F, T, mode, a1=2, a2=2, window=3, stripe=4)
        want = sdpa(q, k, v, m, scale)
        got = oracle.attention_brute(g, mode, q, k, v, scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        got_np, _ = R.attention(q, k, v, m, scale)
        np.testing.assert_allclose(got_np, want, rtol=0, atol=1e-12)
    assert np.all(oracle.attention_brute(g, oracle.SKIP, q, k, v, scale) == 0.0)


def test_dense_reduction(oracle_lib):
    N, F, d = 3, 5, 8
    q, k, v = rand_qkv(N * F, d, seed=7)
    dense = sdpa(q, k, v, np.ones((N * F, N * F), bool), 0.3)
    for a1, a2 in [(N, 1), (N + 2, 1)]:
        got = oracle.attention_brute(oracle.geom(N, F, 0, a1, a2), oracle.SPATIAL, q, k, v, 0.3)
        np.testing.assert_allclose(got, dense, rtol=0, atol=1e-12)
    for a2 in (F, F + 1):
        got = oracle.attention_brute(oracle.geom(N, F, 0, 1, a2), oracle.TEMPORAL, q, k, v, 0.3)
        np.testing.assert_allclose(got, dense, rtol=0, atol=1e-12)


def test_probability_rows(oracle_lib):
    """With V = identity (L <= d) the output row is the attention row itself:
    it sums to one, is exactly zero off the mask, and equals exp(s - max)/sum."""
    N, F, T = 3, 4, 2
    L = T + N * F
    d = 16
    q, k, _ = rand_qkv(L, d, seed=11, scale=2.0)
    v = np.eye(L, d, dtype=np.float32)
    scale = 0.25
    g = oracle.geom(N, F, T, 2, 2, window=3, stripe=4)
    for mode in MODES:
        m = R.dense_mask(N, F, T, mode, a1=2, a2=2, window=3, stripe=4)
        p = oracle.attention_brute(g, mode, q, k, v, scale)[:, :L]
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        assert np.all(p[~m] == 0.0)
        s = (q.astype(np.float64) @ k.T.astype(np.float64)) * scale
        for r in range(L):
            e = np.exp(s[r, m[r]] - s[r, m[r]].max())
            np.testing.assert_allclose(p[r, m[r]], e / e.sum(), rtol=1e-12, atol=0)


def test_constant_values_pass_through(oracle_lib):
    N, F, T, d = 4, 6, 1, 8
    L = T + N * F
    q, k, _ = rand_qkv(L, d, seed=3, scale=3.0)
    c = np.linspace(-2, 2, d).astype(np.float32)
    v = np.tile(c, (L, 1))
    g = oracle.geom(N, F, T, 1, 3, window=2, stripe=5)
    for mode in MODES:
        o = oracle.attention_brute(g, mode, q, k, v, 0.5)
        np.testing.assert_allclose(o, np.tile(c.astype(np.float64), (L, 1)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("N,F,T,a2", [(3, 4, 0, 2), (4, 7, 2, 3), (5, 6, 0, 1), (2, 9, 1, 9)])
def test_permutation_equivariance(oracle_lib, N, F, T, a2):
    """Attention of the token-major tensors under the block band, mapped back
    with the inverse permutation, equals temporal attention in frame-major
    order (the exactness of the layout transformation)."""
    d = 8
    L = T + N * F
    q, k, v = rand_qkv(L, d, seed=5 + a2, scale=1.5)
    g = oracle.geom(N, F, T, 1, a2)
    scale = 1 / np.sqrt(d)
    pi = R.permutation(N, F, T)
    qp, kp, vp = (oracle.permute_rows(g, a) for a in (q, k, v))
    assert np.array_equal(qp[pi], q)
    xp = np.arange(L)
    band = (np.abs((xp[:, None] - T) // N - (xp[None, :] - T) // N) < a2) | (xp[:, None] < T) | (xp[None, :] < T)
    op = sdpa(qp, kp, vp, band, scale)
    back = oracle.permute_rows(g, op, inverse=True)
    nat = oracle.attention_brute(g, oracle.TEMPORAL, q, k, v, scale)
    np.testing.assert_allclose(back, nat, rtol=0, atol=1e-12)
    # the oracle's own token-major predicate gives the same result
    op2 = oracle.attention_brute(g, oracle.TEMPORAL_PERMUTED, qp, kp, vp, scale)
    np.testing.assert_allclose(oracle.permute_rows(g, op2, inverse=True), nat, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,F,T", [(3, 4, 0), (4, 6, 3), (6, 5, 2)])
def test_rows_path_equals_brute(oracle_lib, N, F, T):
    d = 8
    L = T + N * F
    q, k, v = rand_qkv(L, d, seed=N + F + T, scale=1.2)
    g = oracle.geom(N, F, T, 2, 2, window=4, stripe=6)
    rows = np.arange(L)
    for mode in MODES + [oracle.SKIP, oracle.TEMPORAL_PERMUTED]:
        a = oracle.attention_brute(g, mode, q, k, v, 0.4)
        b = oracle.attention_rows(g, mode, q, k, v, 0.4, rows)
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    sub = np.array([L - 1, 0, T + 1])
    np.testing.assert_allclose(oracle.attention_rows(g, oracle.SPATIAL, q, k, v, 0.4, sub),
                               oracle.attention_brute(g, oracle.SPATIAL, q, k, v, 0.4)[sub], rtol=0, atol=1e-12)
