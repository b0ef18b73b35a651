"""svg_sample_rows (host code in the library, no GPU): the sampled query rows
of online profiling are distinct video rows of [T, T + N*F), ascending, and
drawn uniformly without replacement -- every subset of the requested size
equally likely, which a chi-square test over all subsets of small row sets
checks, with each row's inclusion rate checked on a larger set."""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

import sparse_attention_video_svg_amd as svg


def geom(N, F, T=0):
    return svg.Geom(B=1, H=1, d=64, N=N, F=F, T=T, a1=1, a2=1)


@pytest.mark.parametrize("N,F,T,count", [(4, 64, 0, 1), (4, 64, 5, 37), (13, 4080, 0, 531), (33, 3600, 256, 1188),
                                         (2, 3, 1, 6)])
def test_rows_distinct_sorted_in_range(N, F, T, count):
    for seed in (0, 1, 2**63 + 7):
        r = svg.svg_sample_rows(geom(N, F, T), count, seed)
        assert r.dtype == np.int32 and r.shape == (count,)
        assert np.all(np.diff(r) > 0)
        assert r[0] >= T and r[-1] < T + N * F


def test_deterministic_per_seed_and_fresh_across_seeds():
    g = geom(33, 3600)
    a, b, c = (svg.svg_sample_rows(g, 1188, s) for s in (11, 11, 12))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_all_rows_and_no_rows():
    g = geom(4, 64, 7)
    assert np.array_equal(svg.svg_sample_rows(g, 256, 3), np.arange(7, 7 + 256, dtype=np.int32))
    assert svg.svg_sample_rows(g, 0, 3).shape == (0,)


def test_invalid_counts_raise():
    g = geom(4, 64)
    for bad in (-1, 257):
        with pytest.raises(svg.SvgError):
            svg.svg_sample_rows(g, bad, 0)


@pytest.mark.parametrize("n,count", [(6, 3), (5, 2), (7, 1), (7, 6)])
def test_every_subset_equally_likely(n, count):
    g = geom(1, n)
    subsets = {s: i for i, s in enumerate(itertools.combinations(range(n), count))}
    draws = 400 * len(subsets)
    hist = np.zeros(len(subsets))
    for seed in range(draws):
        hist[subsets[tuple(svg.svg_sample_rows(g, count, seed).tolist())]] += 1
    p = stats.chisquare(hist).pvalue
    assert p > 1e-6, (hist, p)


def test_inclusion_rate_uniform_over_rows():
    # 200 rows, 10 drawn: each row in a sample with probability 1/20
    g, count, draws = geom(2, 100), 10, 20000
    hits = np.zeros(200)
    for seed in range(draws):
        hits[svg.svg_sample_rows(g, count, seed)] += 1
    assert hits.sum() == count * draws
    p = stats.chisquare(hits).pvalue
    assert p > 1e-6, p
    # and the first and last rows are not favoured (Floyd's last draws keep j)
    rate = hits / draws
    assert abs(rate[0] - 0.05) < 6 * math.sqrt(0.05 * 0.95 / draws)
    assert abs(rate[-1] - 0.05) < 6 * math.sqrt(0.05 * 0.95 / draws)


def test_inclusion_rate_uniform_sparse_draws():
    # 10 of 1000 rows: the library keeps the drawn set in a hash set for
    # sparse draws (a bitmap otherwise); each row drawn with probability 1/100
    g, count, draws = geom(4, 250), 10, 20000
    hits = np.zeros(1000)
    for seed in range(draws):
        r = svg.svg_sample_rows(g, count, seed)
        assert np.all(np.diff(r) > 0)
        hits[r] += 1
    assert hits.sum() == count * draws
    assert stats.chisquare(hits).pvalue > 1e-6


def test_large_video_small_sample():
    # O(count) work whatever N*F is: 2^29 video rows, 1000 drawn
    r = svg.svg_sample_rows(geom(1 << 14, 1 << 15), 1000, 5)
    assert r.shape == (1000,) and np.all(np.diff(r) > 0) and r[-1] < (1 << 29)
