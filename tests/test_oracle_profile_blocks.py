"""Pins of the oracle's online profiling and key-tile lists (CPU only).

Profiling: planted head types are recovered with a wide margin, heads with
no planted structure fall back to full attention, a dense mask has zero
error (and the tie goes to spatial), the relative error is invariant to the
scale of V, and the C oracle agrees with the independent numpy restatement.
Tile lists: the interval-derived lists equal brute force over elements, and
the longest-first order follows its stated rule.
"""
import numpy as np
import pytest

import oracle
import svg_synth as S
from oracle import ref_numpy as R


@pytest.mark.parametrize("d,N,F,a1,a2", [(64, 6, 96, 2, 12), (128, 5, 120, 1, 20)])
def test_planted_types_recovered(oracle_lib, d, N, F, a1, a2):
    kinds = [S.SPATIAL, S.TEMPORAL, S.SPATIAL, S.TEMPORAL]
    inp = S.small_config(N, F, 0, 4, d, a1, a2, kinds, seed=21)
    g = oracle.geom(N, F, 0, a1, a2)
    rows = S.sample_rows(N, F, 0, 0.05, 4)
    for h in range(4):
        label, st = oracle.profile_head(g, inp["q"][h], inp["k"][h], inp["v"][h], d ** -0.5, rows)
        assert label == kinds[h]
        win, lose = (st[0], st[1]) if kinds[h] == S.SPATIAL else (st[1], st[0])
        assert lose > 30 * max(win, 1e-12) and lose > 0.05


def test_unstructured_falls_back(oracle_lib):
    inp = S.small_config(4, 64, 8, 2, 64, 2, 8, [S.UNSTRUCTURED] * 2, seed=8)
    g = oracle.geom(4, 64, 8, 2, 8)
    rows = S.sample_rows(4, 64, 8, 0.1, 2)
    for h in range(2):
        label, st = oracle.profile_head(g, inp["q"][h], inp["k"][h], inp["v"][h], 0.125, rows)
        assert label == oracle.FULL
        assert min(st[0], st[1]) >= 0.05


def test_dense_mask_zero_error_and_tie(oracle_lib):
    N, F, d = 3, 8, 16
    inp = S.small_config(N, F, 0, 1, d, N, F, [S.UNSTRUCTURED], seed=2)
    g = oracle.geom(N, F, 0, N, F)  # both masks dense
    rows = np.arange(N * F)
    label, st = oracle.profile_head(g, inp["q"][0], inp["k"][0], inp["v"][0], 0.25, rows)
    assert st[0] < 1e-28 and st[1] < 1e-28
    assert label == oracle.SPATIAL  # tie -> spatial


def test_fallback_threshold_and_v_scale(oracle_lib):
    N, F, d = 4, 16, 32
    inp = S.small_config(N, F, 0, 1, d, 1, 3, [S.TEMPORAL], seed=9)
    g = oracle.geom(N, F, 0, 1, 3)
    rows = np.arange(N * F)
    q, k, v = inp["q"][0], inp["k"][0], inp["v"][0]
    lab, st = oracle.profile_head(g, q, k, v, d ** -0.5, rows)
    lab2, st2 = oracle.profile_head(g, q, k, 4.0 * v, d ** -0.5, rows)
    np.testing.assert_allclose(st2[:2], st[:2], rtol=1e-9)
    np.testing.assert_allclose(st2[2], 16.0 * st[2], rtol=1e-12)
    best = min(st[0], st[1])
    # a threshold just above the best error keeps the sparse label, at it falls back
    assert oracle.profile_head(g, q, k, v, d ** -0.5, rows, fallback=best * 1.0001)[0] == lab
    assert oracle.profile_head(g, q, k, v, d ** -0.5, rows, fallback=best)[0] == oracle.FULL


@pytest.mark.parametrize("T", [0, 3])
def test_profile_matches_numpy(oracle_lib, T):
    N, F, d, a1, a2 = 3, 10, 8, 1, 2
    for kinds in ([S.SPATIAL], [S.TEMPORAL], [S.UNSTRUCTURED]):
        inp = S.small_config(N, F, T, 1, d, a1, a2, kinds, seed=31 + T, signal=2.0, noise=0.5)
        g = oracle.geom(N, F, T, a1, a2)
        rows = np.arange(T, T + N * F, 3)
        lab, st = oracle.profile_head(g, inp["q"][0], inp["k"][0], inp["v"][0], 0.3, rows)
        lab_np, st_np = R.profile(inp["q"][0], inp["k"][0], inp["v"][0], N, F, T, a1, a2, 0.3, rows)
        assert lab == lab_np
        np.testing.assert_allclose(st, st_np, rtol=1e-10, atol=1e-300)


@pytest.mark.parametrize("N,F,T,a1,a2", [(4, 12, 0, 1, 2), (5, 9, 3, 2, 3), (3, 16, 2, 1, 16)])
def test_profile_uniform_weights_closed_form(oracle_lib, N, F, T, a1, a2):
    """Q = 0 makes every score equal, so each masked attention output is the
    plain mean of V over the row's active keys (text keys plus the frames
    within a1, or the positions within a2 in every frame).  The statistics
    then follow from means alone: rel_m = sum (mean_m - mean_all)^2 /
    sum mean_all^2 over rows x d, and the third entry mean(mean_all^2)."""
    d = 8
    L = T + N * F
    rng = np.random.default_rng(N * F + T)
    q = np.zeros((L, d), np.float32)
    k = rng.standard_normal((L, d)).astype(np.float32)
    v = (rng.standard_normal((L, d)) + 0.5).astype(np.float32)
    rows = np.arange(T, L, 2)
    g = oracle.geom(N, F, T, a1, a2)
    label, st = oracle.profile_head(g, q, k, v, 0.7, rows)

    def keys(x, mode):
        i, j = divmod(x - T, F)
        ks = list(range(T))
        for x2 in range(T, L):
            i2, j2 = divmod(x2 - T, F)
            if (mode == "s" and abs(i2 - i) < a1) or (mode == "t" and abs(j2 - j) < a2):
                ks.append(x2)
        return ks

    vd = v.astype(np.float64)
    full = np.repeat(vd.mean(axis=0)[None], rows.size, axis=0)
    spat = np.stack([vd[keys(x, "s")].mean(axis=0) for x in rows])
    temp = np.stack([vd[keys(x, "t")].mean(axis=0) for x in rows])
    den = (full ** 2).sum()
    want = [((spat - full) ** 2).sum() / den, ((temp - full) ** 2).sum() / den, (full ** 2).mean()]
    np.testing.assert_allclose(st, want, rtol=1e-12, atol=1e-15)
    rs, rt = want[0], want[1]
    assert label == (oracle.FULL if min(rs, rt) >= 0.05 else oracle.SPATIAL if rs <= rt else oracle.TEMPORAL)


MODES = [oracle.SPATIAL, oracle.TEMPORAL, oracle.FULL, oracle.SKIP, oracle.WINDOW, oracle.STRIPE]


@pytest.mark.parametrize("N,F,T,BM,BN", [(3, 4, 0, 4, 4), (5, 7, 3, 8, 4), (4, 9, 2, 16, 8), (6, 5, 0, 7, 3),
                                          (2, 33, 5, 16, 16)])
def test_blocks_rows_equal_brute(oracle_lib, N, F, T, BM, BN):
    for a1, a2, W, Sp in [(1, 1, 1, 1), (2, 3, 5, 6), (4, 40, 100, 1000)]:
        g = oracle.geom(N, F, T, a1, a2, W, Sp)
        for mode in MODES:
            a = oracle.blocks(g, mode, BM, BN, brute=True)
            b = oracle.blocks(g, mode, BM, BN)
            assert np.array_equal(a, b), (mode, a1, a2)
            if mode == oracle.SKIP:
                assert a.sum() == 0


def test_blocks_cover_the_mask(oracle_lib):
    # every active element lies in a listed tile and no listed tile is empty
    N, F, T, BM, BN = 4, 9, 2, 8, 4
    g = oracle.geom(N, F, T, 2, 3, 5, 7)
    L = T + N * F
    for mode in MODES:
        wm = oracle.TEMPORAL_PERMUTED if mode == oracle.TEMPORAL else mode
        m = oracle.mask_matrix(g, wm)
        bm = oracle.blocks(g, mode, BM, BN)
        pad = np.zeros((bm.shape[0] * BM, bm.shape[1] * BN), np.uint8)
        pad[:L, :L] = m
        per_tile = pad.reshape(bm.shape[0], BM, bm.shape[1], BN).sum(axis=(1, 3))
        assert np.array_equal(per_tile > 0, bm.astype(bool))


def test_head_order_rule(oracle_lib):
    work = np.array([5, 9, 9, 0, 5, 12])
    assert oracle.head_order(work).tolist() == [5, 1, 2, 0, 4, 3]
    assert oracle.head_order(np.zeros(4)).tolist() == [0, 1, 2, 3]
