"""Pins of the oracle's Sparse-vDiT mode search (og_search_head, og_mask_nnz),
against things other than the oracle itself: the literal mask predicates
counted pair by pair, the closed-form pair counts, special cases whose answer
follows from the definition alone (zero values, lambda = 0, a dense window,
the epsilon edge) and the scaling law of the squared error.

Search rule ("Sparse-vDiT" review, "What carries the argument"; referee
report, major comment 1 for the two penalty signs): candidates skip, window,
temporal band, stripe; loss = MSE against full attention + lam * (1 - S)
(Eq. (2)) or + lam * S (Algorithm 1); FULL when every loss exceeds eps."""
import math

import numpy as np
import pytest

import oracle
import svg_synth as S

SKIP, WINDOW, TEMPORAL, STRIPE, FULL = oracle.SKIP, oracle.WINDOW, oracle.TEMPORAL, oracle.STRIPE, oracle.FULL

GEOMS = [
    dict(N=4, F=16, T=0, a1=1, a2=3, window=10, stripe=5),
    dict(N=3, F=20, T=7, a1=2, a2=25, window=100, stripe=70),
    dict(N=5, F=9, T=2, a1=6, a2=4, window=1, stripe=1),
    dict(N=1, F=33, T=0, a1=1, a2=1, window=40, stripe=33),
]


@pytest.mark.parametrize("gk", GEOMS)
def test_mask_nnz_equals_the_predicate_counted_pair_by_pair(gk):
    g = oracle.geom(**gk)
    for mode in (oracle.SPATIAL, TEMPORAL, FULL, WINDOW, STRIPE):
        assert oracle.mask_nnz(g, mode) == int(oracle.mask_matrix(g, mode).sum()), mode
    assert oracle.mask_nnz(g, SKIP) == 0


def closed_form(N, F, T, mode, a1, a2, window, stripe):
    """Pair counts of the masks as sums over block / element diagonals
    (spatial: a1 - 1 frame diagonals each side; temporal: the same over
    positions, N^2 frame pairs; window: |u1 - u2| < W; stripe: keys < stripe),
    plus the dense text rows and columns."""
    NF, L = N * F, T + N * F
    text = L * L - NF * NF
    if mode == oracle.SPATIAL:
        a = min(a1, N)
        v = F * F * (N + 2 * sum(N - k for k in range(1, a)))
    elif mode == TEMPORAL:
        a = min(a2, F)
        v = N * N * (F + 2 * sum(F - k for k in range(1, a)))
    elif mode == WINDOW:
        w = min(window, NF)
        v = NF + 2 * sum(NF - k for k in range(1, w))
    elif mode == STRIPE:
        v = NF * min(stripe, NF)
    else:
        v = NF * NF
    return text + v


@pytest.mark.parametrize("gk", GEOMS + [dict(N=21, F=1560, T=0, a1=2, a2=128, window=1560, stripe=512),
                                       dict(N=33, F=3600, T=256, a1=2, a2=160, window=3600, stripe=512)])
def test_mask_nnz_equals_closed_forms(gk):
    g = oracle.geom(**gk)
    for mode in (oracle.SPATIAL, TEMPORAL, FULL, WINDOW, STRIPE):
        assert oracle.mask_nnz(g, mode) == closed_form(gk["N"], gk["F"], gk["T"], mode, gk["a1"], gk["a2"],
                                                       gk["window"], gk["stripe"])


def planted(kinds, N=6, F=48, T=0, d=64, seed=7, stripe=32):
    inp = S.small_config(N, F, T, len(kinds), d, a1=2, a2=8, kinds=kinds, seed=seed, window=F, stripe=stripe)
    g = oracle.geom(N, F, T, a1=2, a2=8, window=F, stripe=stripe)
    rows = S.sample_rows(N, F, T, 0.25, seed + 1)
    return inp, g, rows


def test_planted_patterns_are_recovered_with_a_small_penalty():
    kinds = [S.WINDOW, S.TEMPORAL, S.STRIPE]
    inp, g, rows = planted(kinds, T=5)
    want = {S.WINDOW: WINDOW, S.TEMPORAL: TEMPORAL, S.STRIPE: STRIPE}
    for h, kd in enumerate(kinds):
        for pen in (0, 1):
            mode, mse, loss, sp = oracle.search_head(g, inp["q"][h], inp["k"][h], inp["v"][h], 1 / 8, rows,
                                                     lam=1e-4, eps=1.0, penalty=pen)
            assert mode == want[kd]
            ci = oracle.SEARCH_CANDIDATES.index(want[kd])
            assert mse[ci] < 1e-4 < 0.05 < min(np.delete(mse, ci))


def test_zero_values_leave_only_the_penalty():
    """V = 0 gives O = 0 for every mask: all MSEs are exactly 0, so Eq. (2)
    picks the sparsest candidate (skip, S = 1) and Algorithm 1 the densest."""
    inp, g, rows = planted([S.WINDOW])
    z = np.zeros_like(inp["v"][0])
    m0, mse, loss, sp = oracle.search_head(g, inp["q"][0], inp["k"][0], z, 1 / 8, rows, lam=0.5, penalty=0)
    assert np.all(mse == 0.0) and m0 == SKIP
    assert sp[0] == 1.0 and np.allclose(loss, 0.5 * (1 - sp))
    m1, mse, loss, sp = oracle.search_head(g, inp["q"][0], inp["k"][0], z, 1 / 8, rows, lam=0.5, penalty=1)
    assert m1 == oracle.SEARCH_CANDIDATES[int(np.argmin(sp))]
    assert np.allclose(loss, 0.5 * sp)


def test_lambda_zero_is_argmin_mse_and_epsilon_edge():
    inp, g, rows = planted([S.FULL, S.STRIPE, S.TEMPORAL])
    for h in range(3):
        mode, mse, loss, sp = oracle.search_head(g, inp["q"][h], inp["k"][h], inp["v"][h], 1 / 8, rows,
                                                 lam=0.0, eps=1e9)
        assert mode == oracle.SEARCH_CANDIDATES[int(np.argmin(mse))]
        assert np.array_equal(loss, mse)
        best = float(loss.min())
        # FULL exactly when every loss is above eps
        m_hi, *_ = oracle.search_head(g, inp["q"][h], inp["k"][h], inp["v"][h], 1 / 8, rows, lam=0.0, eps=best)
        assert m_hi == mode
        m_lo, *_ = oracle.search_head(g, inp["q"][h], inp["k"][h], inp["v"][h], 1 / 8, rows, lam=0.0,
                                      eps=best * (1 - 1e-9) - 1e-300)
        assert m_lo == FULL


def test_mse_scales_with_the_square_of_the_values():
    inp, g, rows = planted([S.FULL])
    _, mse1, _, _ = oracle.search_head(g, inp["q"][0], inp["k"][0], inp["v"][0], 1 / 8, rows, lam=0.0)
    _, mse3, _, _ = oracle.search_head(g, inp["q"][0], inp["k"][0], 3 * inp["v"][0], 1 / 8, rows, lam=0.0)
    assert np.allclose(mse3, 9 * mse1, rtol=1e-12, atol=0)


def test_dense_window_has_zero_error_and_no_sparsity():
    """A window at least as wide as the video keeps every pair: its output is
    full attention over the same keys in the same order, error exactly 0."""
    N, F = 4, 24
    inp = S.small_config(N, F, 0, 1, 64, a1=1, a2=2, kinds=[S.FULL], seed=3, window=N * F)
    g = oracle.geom(N, F, 0, a1=1, a2=2, window=N * F, stripe=8)
    rows = S.sample_rows(N, F, 0, 0.5, 4)
    mode, mse, loss, sp = oracle.search_head(g, inp["q"][0], inp["k"][0], inp["v"][0], 1 / 8, rows, lam=0.0)
    wi = oracle.SEARCH_CANDIDATES.index(WINDOW)
    assert mse[wi] == 0.0 and sp[wi] == 0.0 and mode == WINDOW


def test_skip_error_is_the_mean_square_of_full_attention():
    """The skip candidate's MSE is mean O_full^2, the quantity profiling
    reports as its third statistic (a separate routine)."""
    inp, g, rows = planted([S.TEMPORAL])
    _, mse, _, _ = oracle.search_head(g, inp["q"][0], inp["k"][0], inp["v"][0], 1 / 8, rows)
    _, stats = oracle.profile_head(g, inp["q"][0], inp["k"][0], inp["v"][0], 1 / 8, rows)
    assert math.isclose(mse[0], stats[2], rel_tol=1e-12)


@pytest.mark.parametrize("N,F,T,W,St,a2", [(4, 12, 0, 5, 7, 2), (3, 10, 3, 11, 4, 3), (5, 6, 2, 40, 100, 6)])
def test_uniform_weights_closed_form(N, F, T, W, St, a2):
    """Q = 0 makes every score equal, so each candidate's output is the plain
    mean of V over the row's active keys (text keys plus |u1 - u2| < W for
    the diagonal, |j1 - j2| < a2 for the multi-diagonal, u2 < stripe for the
    stripe) and skip's output is 0.  The MSEs against full attention, the
    sparsities (from the masks' pair counts) and the losses follow."""
    d = 8
    L = T + N * F
    rng = np.random.default_rng(N * F + T + W)
    q = np.zeros((L, d), np.float32)
    k = rng.standard_normal((L, d)).astype(np.float32)
    v = (rng.standard_normal((L, d)) - 0.25).astype(np.float32)
    rows = np.arange(0, L, 2)
    g = oracle.geom(N, F, T, a1=1, a2=a2, window=W, stripe=St)
    lam = 0.3
    mode, mse, loss, sp = oracle.search_head(g, q, k, v, 0.5, rows, lam=lam, eps=10.0)

    def active(x1, x2, c):
        if x1 < T or x2 < T:
            return True
        u1, u2 = x1 - T, x2 - T
        if c == "w":
            return abs(u1 - u2) < W
        if c == "t":
            return abs(u1 % F - u2 % F) < a2
        return u2 < St

    vd = v.astype(np.float64)
    full = np.repeat(vd.mean(axis=0)[None], rows.size, axis=0)
    want_mse, want_sp = [float((full ** 2).mean())], [1.0]
    for c in "wts":
        out = np.stack([vd[[x2 for x2 in range(L) if active(x, x2, c)]].mean(axis=0) for x in rows])
        want_mse.append(float(((out - full) ** 2).mean()))
        nnz = sum(active(x1, x2, c) for x1 in range(L) for x2 in range(L))
        want_sp.append(1.0 - nnz / L ** 2)
    np.testing.assert_allclose(mse, want_mse, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(sp, want_sp, rtol=0, atol=1e-15)
    np.testing.assert_allclose(loss, np.array(want_mse) + lam * (1.0 - np.array(want_sp)), rtol=1e-12, atol=1e-16)
    assert mode == oracle.SEARCH_CANDIDATES[int(np.argmin(loss))]
