"""Workgroup scheduling arithmetic on the CPU (svg_sched.h compiled on its
own with g++): the XCD-aware id remap is a bijection that hands every XCD
runs of consecutive work items for any XCD count, and the key-slice count of
the profiling sweeps follows its rule for any CU count, with the
HunyuanVideo-shaped layer keeping its 8 slices on the MI355X's 256 CUs."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_video_svg_amd", "csrc")

SHIM = r"""
#include "svg_sched.h"
extern "C" {
long long t_xcd_grid(long long total, int nxcd, int run) { return svg::xcd_grid(total, nxcd, run); }
int t_xcd_logical(int w, int nxcd, int run) { return svg::xcd_logical(w, nxcd, run); }
int t_choose_ksplit(long long wgs, long long nkt, long long cus, int cap) {
  return svg::choose_ksplit(wgs, nkt, cus, cap);
}
}
"""


@pytest.fixture(scope="module")
def sched(tmp_path_factory):
    d = tmp_path_factory.mktemp("sched")
    src, lib = d / "shim.cpp", d / "libshim.so"
    src.write_text(SHIM)
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", f"-I{CSRC}", str(src), "-o", str(lib)],
                   check=True)
    L = ctypes.CDLL(str(lib))
    L.t_xcd_grid.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int]
    L.t_xcd_grid.restype = ctypes.c_longlong
    L.t_xcd_logical.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.t_xcd_logical.restype = ctypes.c_int
    L.t_choose_ksplit.argtypes = [ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_int]
    L.t_choose_ksplit.restype = ctypes.c_int
    return L


@pytest.mark.parametrize("nxcd", [1, 2, 4, 8])
@pytest.mark.parametrize("total", [1, 31, 256, 1000, 11160])
def test_xcd_remap_is_a_bijection_with_runs(sched, nxcd, total):
    run = 32
    grid = sched.t_xcd_grid(total, nxcd, run)
    assert grid >= total and grid % (nxcd * run) == 0 and grid - total < nxcd * run
    logical = [sched.t_xcd_logical(w, nxcd, run) for w in range(grid)]
    assert sorted(logical) == list(range(grid))
    # ids w, w + nxcd, w + 2 nxcd, ... run on one XCD: they take consecutive
    # logical items in runs of `run`
    for x in range(nxcd):
        mine = [logical[w] for w in range(x, grid, nxcd)]
        for k in range(0, len(mine), run):
            blk = mine[k:k + run]
            assert blk == list(range(blk[0], blk[0] + run))


def rounds_per_slice(wgs, cus, ks):
    return -(-wgs * ks // cus) / ks


@pytest.mark.parametrize("cus", [32, 64, 256, 304])
@pytest.mark.parametrize("wgs,nkt", [(5 * 24, 1857), (5 * 48, 829), (10 * 24, 1861), (1 * 2, 4)])
def test_ksplit_minimises_rounds(sched, cus, wgs, nkt):
    for cap in (16, 8, 3, 1):
        ks = sched.t_choose_ksplit(wgs, nkt, cus, cap)
        kmax = min(16, nkt, cap)
        assert 1 <= ks <= kmax
        best = min(rounds_per_slice(wgs, cus, k) for k in range(1, kmax + 1))
        assert rounds_per_slice(wgs, cus, ks) <= best + 1e-12


def test_ksplit_unchanged_on_mi355x(sched):
    # HunyuanVideo-shaped layer: 1188 sampled rows in chunks of 256, 24 heads,
    # 1857 key tiles: 8 slices, 960 workgroups = 3.75 rounds of 256 CUs
    assert sched.t_choose_ksplit(5 * 24, 1857, 256, 16) == 8
    # fewer CUs take fewer slices here, within the workspace's 8
    assert sched.t_choose_ksplit(5 * 24, 1857, 64, 8) <= 8
    assert sched.t_choose_ksplit(5 * 24, 1857, 32, 8) <= 8
