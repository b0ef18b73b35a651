"""GPU parity of the whole layer (svg_layer_forward) at the five workload
shapes, in the launch configuration bench.py times (marked gpu).

Per workload: every head's label equals its planted type and the oracle's
label (bit-exact; statistics within 2 %); every head's key-tile ranges, as
svg_build_blocks lays them out for the kernel's tiles, expand to exactly the
oracle's tile bitmap, and the head order equals the oracle's longest-first
order of those bitmaps; outputs of every head on sampled rows (a seeded row in every query
tile, first/last rows, band edges, seeded picks) within max-abs 2e-2 / RMS 2e-3 (bf16) or
1e-5 (fp32) of the oracle; explicit and virtual layout transformation give
identical bits; a rerun is bit-identical.  Shapes:
  0  tiny fp32        4 x 64 tokens, 2 heads, d 64, all rows profiled
  1  CogVideoX-like   13 x 4080, 48 heads, d 64
  2  HunyuanVideo-like 33 x 3600, 24 heads, d 128
  3  as 2 + 256 text tokens, 10 spatial / 9 temporal / 5 unstructured, 4 calls
  4  Sparse-vDiT set  21 x 1560, 40 heads, d 128, fixed modes, no profiling
"""
import numpy as np
import pytest

import oracle
import sparse_attention_video_svg_amd as svg
import svg_synth as S
from helpers import block_bitmap_from_ranges, check_close, ogeom, rows_per_tile, sample_check_rows, scale_of

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PLANT_TO_LABEL = {S.SPATIAL: svg.SPATIAL, S.TEMPORAL: svg.TEMPORAL, S.UNSTRUCTURED: svg.FULL}


def geom_of(c):
    return svg.Geom(B=1, H=c["H"], d=c["d"], N=c["N"], F=c["F"], T=c["T"], a1=c["a1"], a2=c["a2"],
                    window=c.get("window", c["F"]), stripe=c.get("stripe", 512))


def run_layer(g, q, k, v, rows, modes_in, flags, out_dtype):
    din = svg.BF16 if q.dtype == torch.bfloat16 else svg.F32
    n_rows = 0 if rows is None else rows.numel()
    ws = svg.alloc_workspace(g, din, n_rows if modes_in is None else 0, flags)
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    labels = torch.full((g.H,), -1, dtype=torch.int32, device="cuda")
    stats = torch.zeros(g.H * 3, dtype=torch.float32, device="cuda")
    svg.svg_layer_forward(g, q, k, v, o, ws, rows=rows, labels_out=labels, stats_out=stats, modes_in=modes_in,
                          flags=flags)
    torch.cuda.synchronize()
    return o, labels.cpu().numpy(), stats.cpu().numpy().reshape(g.H, 3)


def band_edge_rows(g, label):
    """Rows at the edges of the frame runs (spatial) or of the position band."""
    T, F, N = g.T, g.F, g.N
    rows = []
    for i in (0, 1, N // 2, N - 1):
        rows += [T + i * F, T + i * F + F - 1]
    if label == svg.TEMPORAL:
        rows += [T + j for j in (0, g.a2 - 1, g.a2, F - 1)]
    return rows


CASES = [(0, 0), (1, 0), (2, 0), (3, 0), (3, 1), (3, 2), (3, 3), (4, 0)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,call", CASES)
def test_layer_parity(cfg, call):
    c = S.WORKLOADS[cfg]
    print(f"\n[workload {cfg} call {call}: {c['name']}]", flush=True)
    inp = S.make_inputs(cfg, call=call)
    g = geom_of(c)
    bf16 = c["dtype"] == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    q, k, v = (torch.from_numpy(inp[n]).cuda().to(tdt)[None] for n in "qkv")
    profile = inp["rows"] is not None
    rows = torch.from_numpy(inp["rows"]).cuda() if profile else None
    modes_in = None if profile else torch.from_numpy(inp["kinds"].astype(np.int32)).cuda()
    o_e, lab, st = run_layer(g, q, k, v, rows, modes_in, 0, tdt)
    o_v, lab_v, st_v = run_layer(g, q, k, v, rows, modes_in, svg.VIRTUAL_PERMUTE, tdt)
    o_r, lab_r, _ = run_layer(g, q, k, v, rows, modes_in, svg.VIRTUAL_PERMUTE, tdt)
    assert np.array_equal(lab, lab_v) and np.array_equal(lab, lab_r)
    assert np.array_equal(st, st_v)
    assert torch.equal(o_e.view(torch.int16) if bf16 else o_e.view(torch.int32),
                       o_v.view(torch.int16) if bf16 else o_v.view(torch.int32)), "explicit != virtual"
    assert torch.equal(o_v, o_r), "rerun not bit-identical"
    if profile:
        want = np.array([PLANT_TO_LABEL[int(x)] for x in inp["kinds"]])
        assert np.array_equal(lab, want), (lab, want)
    else:
        assert np.array_equal(lab, inp["kinds"])
    og = ogeom(g)
    sc = scale_of(g)
    # key-tile lists of every head, in the kernel's tiles, against the
    # oracle's element-level bitmap; head order against the oracle's
    BM, BN = svg.svg_tile_config(svg.BF16 if bf16 else svg.F32, g.d)
    nq, nk = -(-g.L // BM), -(-g.L // BN)
    modes_dev = torch.from_numpy(lab.astype(np.int32)).cuda()
    ranges = torch.full((g.H * nq * 4,), -1, dtype=torch.int32, device="cuda")
    order = torch.full((g.H,), -1, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes_dev, BM, BN, ranges, order)
    torch.cuda.synchronize()
    rg = ranges.cpu().numpy().reshape(g.H, nq * 4)
    work = np.zeros(g.H, dtype=np.int64)
    for h in range(g.H):
        got = block_bitmap_from_ranges(rg[h], nq, nk)
        want = oracle.blocks(og, int(lab[h]), BM, BN)
        assert np.array_equal(got, want), (f"config {cfg} head {h} (mode {lab[h]}): tile lists differ in "
                                           f"{int((got != want).sum())} of {nq * nk} tiles")
        work[h] = int(want.sum())
    assert np.array_equal(order.cpu().numpy(), oracle.head_order(work)), "head order"
    print(f"  tile lists: {g.H} heads bit-exact ({nq} x {nk} tiles each), head order equal", flush=True)
    # the oracle's profiling of every head
    if profile:
        for h in range(g.H):
            ref_label, ref_stats = oracle.profile_head(og, inp["q"][h], inp["k"][h], inp["v"][h], sc,
                                                       inp["rows"].astype(np.int64))
            assert lab[h] == ref_label, (h, lab[h], ref_label)
            np.testing.assert_allclose(st[h], ref_stats, rtol=2e-2, atol=1e-4)
        print(f"  labels: all {g.H} heads equal the oracle's", flush=True)
    # outputs of every head on sampled rows
    out = o_e[0].float().cpu().numpy()
    worst = (0.0, 0.0)
    inv = oracle.perm_inv_index(og) if cfg != 0 else None  # token-major row -> natural row
    for h in range(g.H):
        if cfg == 0:
            check = np.arange(g.L)
        else:
            # temporal heads run in token-major order: a row in each of those query tiles
            tiles = rows_per_tile(g.L, BM, seed=h)
            if lab[h] == svg.TEMPORAL:
                tiles = inv[tiles]
            check = np.union1d(sample_check_rows(g.L, g.T, band_edge_rows(g, lab[h]), n=24, seed=h), tiles)
        ref = oracle.attention_rows(og, int(lab[h]), inp["q"][h], inp["k"][h], inp["v"][h], sc, check)
        mx, rms = check_close(out[h][check], ref, "bf16" if bf16 else "f32", what=f"config {cfg} head {h}")
        worst = (max(worst[0], mx), max(worst[1], rms))
    print(f"  outputs: worst max-abs {worst[0]:.3e}, worst rms {worst[1]:.3e}", flush=True)
