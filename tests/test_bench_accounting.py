"""CPU checks of bench.py's bookkeeping: the closed-form pair counts that
turn kernel time into effective TFLOP/s equal the oracle's mask sums."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("N,F,T", [(3, 4, 0), (4, 7, 3), (5, 6, 2), (2, 9, 0)])
def test_pair_count_matches_oracle_masks(oracle_lib, N, F, T):
    for a1, a2, W, S in [(1, 1, 1, 1), (2, 3, 4, 5), (9, 9, 100, 1000)]:
        g = oracle.geom(N, F, T, a1, a2, W, S)
        for mode in (oracle.SPATIAL, oracle.TEMPORAL, oracle.FULL, oracle.SKIP, oracle.WINDOW, oracle.STRIPE):
            want = int(oracle.mask_matrix(g, mode).sum())
            assert bench.pair_count(N, F, T, mode, a1, a2, W, S) == want, (mode, a1, a2)


def test_config2_density():
    # spatial 97/1089 and temporal ~8.66 % of 118,800^2 pairs, as the closed forms give
    n = 33 * 3600
    sp = bench.pair_count(33, 3600, 0, 0, a1=2)
    tp = bench.pair_count(33, 3600, 0, 1, a2=160)
    assert sp == 1_257_120_000 and tp == 1_222_903_440
    assert abs(sp / n ** 2 - 97 / 1089) < 1e-12


def test_bench_refuses_several_gpus():
    import subprocess, sys, os
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
