"""Host-side argument checks of the Python binding: the always-on metadata
checks of small device vectors (dtype, contiguity, length) and the DEBUG
content checks of sampled rows, modes, tile ranges and head order.  Pure host
logic (no library call, no GPU)."""
import pytest
import torch

import sparse_attention_video_svg_amd as svg

G = svg.Geom(B=1, H=3, d=64, N=4, F=50, T=6, a1=1, a2=5)   # L = 206


def test_check_vec_dtype_contiguity_length():
    with pytest.raises(TypeError, match="int32"):
        svg._check_vec(torch.zeros(4, dtype=torch.int64), "rows", torch.int32, 1)
    with pytest.raises(ValueError, match="contiguous"):
        svg._check_vec(torch.zeros(8, dtype=torch.int32)[::2], "modes", torch.int32, 1)
    with pytest.raises(ValueError, match="needs 3"):
        svg._check_vec(torch.zeros(2, dtype=torch.int32), "labels", torch.int32, 3)
    with pytest.raises(ValueError, match="device"):
        svg._check_vec(torch.zeros(3, dtype=torch.int32), "labels", torch.int32, 3)
    with pytest.raises(ValueError, match="required"):
        svg._check_vec(None, "modes", torch.int32, 3)
    svg._check_vec(None, "modes_in", torch.int32, 3, optional=True)


@pytest.mark.parametrize("rows,ok", [
    ([6, 7, 100, 205], True),
    ([6], True),
    ([5, 7], False),          # a text row
    ([7, 206], False),        # past the end
    ([9, 8], False),          # descending
    ([9, 9, 10], False),      # repeated
    ([], False),
])
def test_debug_rows(rows, ok):
    t = torch.tensor(rows, dtype=torch.int32)
    if ok:
        svg._debug_rows(G, t)
    else:
        with pytest.raises(ValueError):
            svg._debug_rows(G, t)


def test_debug_modes():
    svg._debug_modes(G, torch.tensor([svg.SPATIAL, svg.STRIPE, svg.SKIP], dtype=torch.int32))
    for bad in ([0, 6, 1], [-1, 0, 0]):
        with pytest.raises(ValueError, match="not a mode"):
            svg._debug_modes(G, torch.tensor(bad, dtype=torch.int32))


def test_debug_tiles():
    BM, BN = 128, 64
    nq, nk = -(-G.L // BM), -(-G.L // BN)          # 2 query tiles, 4 key tiles
    good = [[0, 4, 0, 0], [0, 1, 2, 4]] * 3          # one range; text range then band
    svg._debug_tiles(G, BM, BN, torch.tensor(good, dtype=torch.int32).flatten(),
                     torch.tensor([2, 0, 1], dtype=torch.int32))
    for bad in ([2, 1, 0, 0], [0, 3, 2, 4], [0, 5, 0, 0], [0, 1, 3, 5], [-1, 1, 0, 0]):
        r = torch.tensor([bad] + good[1:], dtype=torch.int32).flatten()
        with pytest.raises(ValueError, match="ranges entry 0"):
            svg._debug_tiles(G, BM, BN, r, torch.tensor([0, 1, 2], dtype=torch.int32))
    for order in ([0, 0, 1], [0, 1, 3]):
        with pytest.raises(ValueError, match="permutation"):
            svg._debug_tiles(G, BM, BN, torch.tensor(good, dtype=torch.int32).flatten(),
                             torch.tensor(order, dtype=torch.int32))
    assert nq * 4 * G.H == len(good) * 4 and nk == 4
