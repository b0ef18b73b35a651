"""Pins of the oracle's SVG2 mode (oracle/svg2.py) against the definitions
and against routines other than itself: the Lloyd invariants (labels are
the nearest previous centroids by brute force, centroids the means of their
tokens), the degenerate cluster counts, the stable permutation, the
selection's limits (p -> 1 takes every non-empty cluster, small p only the
best one), and the attention reducing to the oracle's dense attention (a
separate C routine) when every cluster is selected."""
import math

import numpy as np
import pytest

import oracle
from oracle import svg2


def mixture(L, d, G, seed, spread=4.0, noise=0.3):
    rng = np.random.default_rng(seed)
    centers = rng.standard_normal((G, d)) * spread
    g = rng.integers(0, G, L)
    return centers[g] + noise * rng.standard_normal((L, d)), g, centers


def test_lloyd_invariants():
    x, _, _ = mixture(300, 16, 7, 0)
    C = 9
    mu0 = svg2.strided_init(x, C)
    labels, mu, counts = svg2.kmeans(x, C, 1)
    # one iteration: labels are the brute-force nearest initial centroids
    for t in range(x.shape[0]):
        dist = [float(np.sum((x[t] - mu0[c]) ** 2)) for c in range(C)]
        assert labels[t] == dist.index(min(dist))
    for c in range(C):
        if counts[c]:
            assert np.allclose(mu[c], x[labels == c].mean(axis=0), rtol=0, atol=1e-12)
        else:
            assert np.array_equal(mu[c], mu0[c])
    assert counts.sum() == x.shape[0]


def test_separated_mixture_is_recovered_from_its_centres():
    x, g, centers = mixture(500, 32, 6, 1)
    labels, mu, counts = svg2.kmeans(x, 6, 3, init=centers + 0.1)
    assert np.array_equal(labels, g)
    assert np.allclose(mu, np.array([x[g == c].mean(axis=0) for c in range(6)]))


def test_degenerate_cluster_counts():
    x, _, _ = mixture(40, 8, 3, 2)
    labels, mu, _ = svg2.kmeans(x, 40, 2)  # one cluster per token
    assert np.array_equal(labels, np.arange(40)) and np.allclose(mu, x)
    labels, mu, counts = svg2.kmeans(x, 1, 2)
    assert np.all(labels == 0) and counts[0] == 40 and np.allclose(mu[0], x.mean(axis=0))


def test_fixed_point():
    x, _, _ = mixture(400, 16, 5, 3)
    l1, m1, _ = svg2.kmeans(x, 5, 30)
    l2, m2, _ = svg2.kmeans(x, 5, 1, init=m1)
    assert np.array_equal(l1, l2) and np.allclose(m1, m2)


def test_permutation_is_stable_and_grouped():
    rng = np.random.default_rng(4)
    labels = rng.integers(0, 7, 200)
    perm, start = svg2.permutation(labels, 7)
    assert sorted(perm.tolist()) == list(range(200))
    assert start[0] == 0 and start[-1] == 200
    for c in range(7):
        seg = perm[start[c]:start[c + 1]]
        assert np.all(labels[seg] == c) and np.all(np.diff(seg) > 0)


def test_scores_and_top_p_limits():
    rng = np.random.default_rng(5)
    mq, mk = rng.standard_normal((6, 16)), rng.standard_normal((9, 16))
    counts = rng.integers(0, 30, 9)
    counts[3] = 0
    P = svg2.cluster_scores(mq, mk, counts, 0.5)
    assert np.allclose(P.sum(axis=1), 1.0) and np.all(P[:, 3] == 0)
    # P is proportional to n_b exp(z_ab) (a restatement via logs)
    z = 0.5 * mq @ mk.T
    nz = counts > 0
    lr = np.log(P[:, nz]) - (np.log(counts[nz])[None, :] + z[:, nz])
    assert np.allclose(lr - lr[:, :1], 0.0, atol=1e-12)
    every = svg2.top_p(P, counts, 1.0 + 1e-9)
    assert np.array_equal(every, np.broadcast_to(counts > 0, every.shape))
    one = svg2.top_p(P, counts, 1e-9)
    assert np.all(one.sum(axis=1) == 1) and np.array_equal(np.argmax(one, axis=1), np.argmax(P, axis=1))
    mid = svg2.top_p(P, counts, 0.6)
    for a in range(6):  # the selected mass reaches p, dropping the smallest selected one does not
        s = P[a][mid[a]]
        assert s.sum() >= 0.6 and s.sum() - s.min() < 0.6


def test_attention_with_every_cluster_is_dense_attention():
    rng = np.random.default_rng(6)
    L, d = 96, 32
    q, k, v = (rng.standard_normal((L, d)).astype(np.float32) for _ in range(3))
    lq, lk = rng.integers(0, 5, L), rng.integers(0, 4, L)
    sel = np.ones((5, 4), dtype=bool)
    rows = np.arange(L)
    got = svg2.attention_rows(q, k, v, lq, lk, sel, 1 / math.sqrt(d), rows)
    g = oracle.geom(1, L)
    want = oracle.attention_rows(g, oracle.FULL, q, k, v, 1 / math.sqrt(d), rows)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_attention_masks_by_cluster_pair():
    """With a block-diagonal selection every row attends only to its own
    cluster's keys: equal to dense attention restricted to those keys."""
    rng = np.random.default_rng(7)
    L, d = 64, 16
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    lab = rng.integers(0, 3, L)
    sel = np.eye(3, dtype=bool)
    got = svg2.attention_rows(q, k, v, lab, lab, sel, 0.25, np.arange(L))
    for x in range(L):
        keys = np.flatnonzero(lab == lab[x])
        s = 0.25 * k[keys] @ q[x]
        w = np.exp(s - s.max())
        assert np.allclose(got[x], w @ v[keys] / w.sum())
