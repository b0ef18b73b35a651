"""Pins of the oracle's masks and layout transformation (CPU only).

Every check compares the oracle with something other than itself: matrices
drawn by hand (tests/golden), the closed-form nonzero counts, the structural
facts the pages state (block band, 2N-1 slashes, dense limits), an
independent numpy broadcast of the definitions, and brute force.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import ref_numpy as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    rows = [ln.strip() for ln in open(os.path.join(GOLD, name)) if ln.strip() and not ln.startswith("#")]
    return rows


def golden_matrix(name):
    return np.array([[int(ch) for ch in r] for r in load_golden(name)], dtype=np.uint8)


@pytest.mark.parametrize("name,N,F,T,mode,a1,a2", [
    ("spatial_N3_F4_a2.txt", 3, 4, 0, oracle.SPATIAL, 2, 1),
    ("temporal_N3_F4_a2.txt", 3, 4, 0, oracle.TEMPORAL, 1, 2),
    ("spatial_N3_F4_a2_T2.txt", 3, 4, 2, oracle.SPATIAL, 2, 1),
    ("temporal_permuted_N3_F4_a2.txt", 3, 4, 0, oracle.TEMPORAL_PERMUTED, 1, 2),
])
def test_golden_masks(oracle_lib, name, N, F, T, mode, a1, a2):
    g = oracle.geom(N, F, T, a1, a2)
    want = golden_matrix(name)
    got = oracle.mask_matrix(g, mode)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_golden_permutation(oracle_lib):
    want = np.array([int(t) for t in load_golden("perm_N3_F4.txt")[0].split()])
    g = oracle.geom(3, 4)
    assert np.array_equal(oracle.perm_index(g), want)
    assert np.array_equal(R.permutation(3, 4, 0), want)


def spatial_count(N, F, a1):
    # closed form F^2 (N + 2 sum_{k=1}^{a1-1} (N-k)), a1 clipped to N
    a = min(a1, N)
    return F * F * (N + 2 * sum(N - k for k in range(1, a)))


def temporal_count(N, F, a2):
    a = min(a2, F)
    return N * N * (F + 2 * sum(F - k for k in range(1, a)))


SHAPES = [(1, 5), (2, 3), (3, 4), (4, 6), (5, 8), (3, 16), (6, 5)]


@pytest.mark.parametrize("N,F", SHAPES)
def test_closed_form_counts(oracle_lib, N, F):
    for a1 in range(1, N + 3):
        g = oracle.geom(N, F, 0, a1, 1)
        m = oracle.mask_matrix(g, oracle.SPATIAL)
        assert int(m.sum()) == spatial_count(N, F, a1)
        assert int(R.dense_mask(N, F, 0, R.SPATIAL, a1=a1).sum()) == spatial_count(N, F, a1)
    for a2 in range(1, F + 3):
        g = oracle.geom(N, F, 0, 1, a2)
        m = oracle.mask_matrix(g, oracle.TEMPORAL)
        assert int(m.sum()) == temporal_count(N, F, a2)
        assert int(R.dense_mask(N, F, 0, R.TEMPORAL, a2=a2).sum()) == temporal_count(N, F, a2)


@pytest.mark.parametrize("N,F", SHAPES)
def test_dense_limits_and_symmetry(oracle_lib, N, F):
    L = N * F
    for a1 in (N, N + 1):
        assert oracle.mask_matrix(oracle.geom(N, F, 0, a1, 1), oracle.SPATIAL).sum() == L * L
    for a2 in (F, F + 3):
        assert oracle.mask_matrix(oracle.geom(N, F, 0, 1, a2), oracle.TEMPORAL).sum() == L * L
    g = oracle.geom(N, F, 2, 2, 2, window=3, stripe=4)
    for mode in (oracle.SPATIAL, oracle.TEMPORAL, oracle.WINDOW, oracle.FULL):
        m = oracle.mask_matrix(g, mode)
        assert np.array_equal(m, m.T)
    st = oracle.mask_matrix(g, oracle.STRIPE)
    assert not np.array_equal(st, st.T) or L + 2 <= 4


@pytest.mark.parametrize("N,F", SHAPES)
def test_oracle_matches_numpy_broadcast(oracle_lib, N, F):
    for T in (0, 3):
        g = oracle.geom(N, F, T, 2, 2, window=F, stripe=5)
        for mode in (oracle.SPATIAL, oracle.TEMPORAL, oracle.FULL, oracle.SKIP, oracle.WINDOW, oracle.STRIPE):
            want = R.dense_mask(N, F, T, mode, a1=2, a2=2, window=F, stripe=5)
            assert np.array_equal(oracle.mask_matrix(g, mode).astype(bool), want), mode


def test_block_band_structure(oracle_lib):
    # "main diagonal plus +-(a1-1) diagonals" are block (frame) diagonals
    for N, F in [(5, 3), (6, 4), (4, 7)]:
        for a1 in range(1, N + 2):
            m = oracle.mask_matrix(oracle.geom(N, F, 0, a1, 1), oracle.SPATIAL)
            diag = set()
            for x1, x2 in zip(*np.nonzero(m)):
                diag.add(x1 // F - x2 // F)
            assert diag == set(range(-(min(a1, N) - 1), min(a1, N)))
            # each listed frame pair is a full F x F block
            blocks = m.reshape(N, F, N, F).sum(axis=(1, 3))
            assert set(np.unique(blocks)) <= {0, F * F}


def test_temporal_slashes(oracle_lib):
    # 2N-1 slanted diagonals at offsets x1 - x2 = k F, each of width a2
    for N, F, a2 in [(3, 8, 2), (4, 10, 3), (5, 9, 1), (2, 12, 4)]:
        m = oracle.mask_matrix(oracle.geom(N, F, 0, 1, a2), oracle.TEMPORAL)
        offs = {int(x1) - int(x2) for x1, x2 in zip(*np.nonzero(m))}
        slashes = {int(np.floor(o / F + 0.5)) for o in offs}
        assert slashes == set(range(-(N - 1), N))
        for k in slashes:
            width = {o - k * F for o in offs if int(np.floor(o / F + 0.5)) == k}
            assert width == set(range(-(a2 - 1), a2))


def test_slash_form_readings(oracle_lib):
    """The page's third form of the temporal mask, read two ways.

    Reading adopted: k ranges over -(N-1)..N-1 (2N-1 values) and each slash is
    clipped to its F x F block -> identical to the mod form.  Unclipped, the
    slash form is a strict superset by exactly (N^2-1) a2 (a2-1) pairs when
    2 a2 <= F; the literal 0 <= k < 2N-1 range is not even symmetric."""
    for N, F, a2 in [(2, 4, 2), (3, 5, 2), (3, 8, 3), (4, 6, 2), (5, 8, 4)]:
        mod = oracle.mask_matrix(oracle.geom(N, F, 0, 1, a2), oracle.TEMPORAL).astype(bool)
        L = N * F
        x1 = np.arange(L)[:, None]
        x2 = np.arange(L)[None, :]
        clipped = np.zeros((L, L), bool)
        glob = np.zeros((L, L), bool)
        literal = np.zeros((L, L), bool)
        for k in range(-(N - 1), N):
            near = np.abs((x1 - x2) - k * F) < a2
            clipped |= near & ((x1 // F - x2 // F) == k)
            glob |= near
        for k in range(0, 2 * N - 1):
            literal |= np.abs((x1 - x2) - k * F) < a2
        assert np.array_equal(clipped, mod)
        assert np.all(glob >= mod)
        if 2 * a2 <= F:
            assert int(glob.sum() - mod.sum()) == (N * N - 1) * a2 * (a2 - 1)
        assert not np.array_equal(literal, literal.T)


@pytest.mark.parametrize("N,F,T", [(3, 4, 0), (5, 7, 0), (4, 6, 3), (1, 9, 2), (7, 1, 1)])
def test_permutation_bijection_and_band(oracle_lib, N, F, T):
    g = oracle.geom(N, F, T, 1, 2)
    pi = oracle.perm_index(g)
    pinv = oracle.perm_inv_index(g)
    L = T + N * F
    assert sorted(pi.tolist()) == list(range(L))
    assert np.array_equal(pinv[pi], np.arange(L))
    assert np.array_equal(pi, R.permutation(N, F, T))
    # row permutation of data and its inverse are exact
    data = np.arange(L * 3, dtype=np.uint16).reshape(L, 3)
    fw = oracle.permute_rows(g, data)
    assert np.array_equal(fw[pi], data)
    assert np.array_equal(oracle.permute_rows(g, fw, inverse=True), data)
    # the temporal mask in token-major order is the block band |floor(u1/N)-floor(u2/N)| < a2
    for a2 in range(1, F + 2):
        g2 = oracle.geom(N, F, T, 1, a2)
        nat = R.dense_mask(N, F, T, R.TEMPORAL, a2=a2)
        permuted = np.zeros_like(nat)
        permuted[np.ix_(pi, pi)] = nat
        xp = np.arange(L)
        up1, up2 = (xp[:, None] - T), (xp[None, :] - T)
        band = (np.abs(up1 // N - up2 // N) < a2) | (xp[:, None] < T) | (xp[None, :] < T)
        assert np.array_equal(permuted, band)
        assert np.array_equal(oracle.mask_matrix(g2, oracle.TEMPORAL_PERMUTED).astype(bool), band)


@pytest.mark.parametrize("N,F,T", [(3, 4, 0), (4, 6, 3), (5, 3, 2), (2, 9, 0)])
def test_row_intervals_match_predicate(oracle_lib, N, F, T):
    for a1, a2, W, S in [(1, 1, 1, 1), (2, 2, 3, 4), (3, 5, 7, 100), (9, 9, 100, 2)]:
        g = oracle.geom(N, F, T, a1, a2, W, S)
        L = T + N * F
        for mode in (oracle.SPATIAL, oracle.TEMPORAL, oracle.FULL, oracle.SKIP, oracle.WINDOW,
                     oracle.STRIPE, oracle.TEMPORAL_PERMUTED):
            m = oracle.mask_matrix(g, mode)
            for x1 in range(L):
                iv = oracle.row_intervals(g, mode, x1)
                got = np.zeros(L, np.uint8)
                prev = -1
                for lo, hi in iv:
                    assert lo < hi and lo > prev  # sorted, disjoint, non-touching
                    prev = hi
                    got[lo:hi] = 1
                assert np.array_equal(got, m[x1]), (mode, x1)


def test_row_intervals_never_truncate(oracle_lib):
    """A temporal row with many frames has one interval per frame: more
    frames than any fixed buffer must still come out whole, and a capacity
    that is too small is an error, not a silently shortened list."""
    N, F, T, a2 = 5000, 4, 3, 1
    g = oracle.geom(N, F, T, 1, a2)
    assert oracle.max_intervals(g) == N + 1
    x1 = T + 7 * F + 2  # frame 7, position 2
    iv = oracle.row_intervals(g, oracle.TEMPORAL, x1)
    assert len(iv) == N + 1  # the text columns, then position 2 of every frame
    assert iv[0] == (0, T)
    assert all(iv[1 + i] == (T + i * F + 2, T + i * F + 3) for i in range(N))
    with pytest.raises(ValueError):
        oracle.row_intervals(g, oracle.TEMPORAL, x1, max_n=N)
    # whole-map count against the closed form N^2 (F + 2 sum_{k<a2} (F-k)) plus the dense text rows/columns
    g0 = oracle.geom(N, F, 0, 1, a2)
    assert oracle.mask_nnz(g0, oracle.TEMPORAL) == N * N * F
    L = T + N * F
    assert oracle.mask_nnz(g, oracle.TEMPORAL) == N * N * F + T * L + N * F * T
