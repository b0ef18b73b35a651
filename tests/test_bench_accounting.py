"""CPU checks of bench.py's bookkeeping: the closed-form pair counts that
turn kernel time into effective TFLOP/s equal the oracle's mask sums."""
import os

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


@pytest.mark.parametrize("N,F,T", [(4, 7, 3), (5, 6, 0), (3, 20, 11)])
def test_search_key_count_matches_oracle_intervals(oracle_lib, N, F, T):
    """The mode search's work figure: keys per sampled row over the four masks
    it sweeps (full, window, temporal band, stripe) equals the oracle's
    per-row intervals summed."""
    import sparse_attention_video_svg_amd as svg
    for a1, a2, W, S in [(1, 2, 3, 4), (2, 9, 50, 2)]:
        g = oracle.geom(N, F, T, a1, a2, W, S)
        geom = svg.Geom(B=1, H=1, d=64, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=S)
        rows = np.arange(T, T + N * F, 3, dtype=np.int32)
        want = 0
        for x in rows:
            for mode in (oracle.FULL, oracle.WINDOW, oracle.TEMPORAL, oracle.STRIPE):
                want += sum(h - l for l, h in oracle.row_intervals(g, mode, int(x)))
        assert bench.search_keys(geom, rows) == want


def test_traffic_record_is_guarded_by_source_hash(tmp_path, monkeypatch):
    """A committed counter record feeds roofline.traffic only while the hash of
    its kernel's sources is the one it was taken at, and only for its own
    kernel, workload and layout."""
    (tmp_path / "profiles").mkdir()
    name = bench.TRAFFIC_RECORDS[("k_attn_bf16", 2, "explicit")]
    sha = bench.source_sha256("k_attn_bf16")

    def write(kernel, digest):
        (tmp_path / "profiles" / name).write_text(
            f"# summary\n\n- record_kernel: {kernel}\n- record_source_sha256: {digest}\n"
            "- record_traffic_bytes_per_dispatch: 7.5e+09\n")

    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    write("k_attn_bf16", sha)
    assert bench.recorded_traffic("k_attn_bf16", 2, "explicit") == 7.5e9
    assert bench.recorded_traffic("k_attn_bf16", 2, "virtual") is None
    assert bench.recorded_traffic("k_attn_bf16", 0, "explicit") is None
    write("k_attn_bf16", "0" * 64)
    assert bench.recorded_traffic("k_attn_bf16", 2, "explicit") is None
    write("k_attn_fp8", sha)
    assert bench.recorded_traffic("k_attn_bf16", 2, "explicit") is None


def test_kernel_source_sets_exist_and_differ():
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.isfile(os.path.join(bench.CSRC, f)), (kernel, f)
    shas = {k: bench.source_sha256(k) for k in bench.KERNEL_SOURCES}
    assert len(set(shas.values())) == len(shas)
    assert bench.source_sha256("k_attn_fp8pv") == shas["k_attn_fp8"]
