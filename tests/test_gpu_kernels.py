"""GPU parity of every kernel family against the CPU oracle on small shapes
that still span several tiles and end in ragged tails (marked gpu).

Bars: layout transformation, tile lists and head labels bit-exact; attention
max-abs <= 2e-2 and RMS <= 2e-3 for bf16 inputs, max-abs <= 1e-5 for fp32."""
import numpy as np
import pytest

import oracle
import sparse_attention_video_svg_amd as svg
import svg_synth as S
from helpers import (block_bitmap_from_ranges, check_close, ogeom, scale_of, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MODES6 = [svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.SKIP, svg.WINDOW, svg.STRIPE]


def planted_kind(mode):
    return {svg.SPATIAL: S.SPATIAL, svg.TEMPORAL: S.TEMPORAL, svg.FULL: S.FULL, svg.SKIP: S.FULL,
            svg.WINDOW: S.WINDOW, svg.STRIPE: S.STRIPE}[mode]


@pytest.mark.parametrize("dt,N,F,T,d,pad", [
    ("bf16", 5, 37, 3, 64, 0), ("bf16", 7, 9, 0, 128, 8), ("bf16", 33, 20, 70, 128, 0),
    ("f32", 3, 40, 5, 64, 4), ("f32", 4, 64, 0, 128, 0)])
def test_layout_permute_bit_exact(dt, N, F, T, d, pad):
    B, H = 2, 3
    g = svg.Geom(B=B, H=H, d=d, N=N, F=F, T=T)
    L = g.L
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    idt = torch.int16 if dt == "bf16" else torch.int32
    gen = torch.Generator().manual_seed(N * 1000 + F)
    base = torch.randint(-30000, 30000, (B, H, L, d + pad), generator=gen, dtype=torch.int32).to(idt)
    src = base.cuda().view(tdt)[..., :d]
    dst = torch.full((B, H, L, d), 7, dtype=idt).cuda().view(tdt)
    modes = torch.tensor([svg.TEMPORAL, svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.TEMPORAL, svg.SKIP],
                         dtype=torch.int32).cuda()
    svg.svg_layout_permute(g, src, dst, modes=modes)
    back = torch.full_like(dst, 0)
    svg.svg_layout_permute(g, dst, back, modes=modes, inverse=True)
    allp = torch.empty_like(dst)
    svg.svg_layout_permute(g, src, allp)
    torch.cuda.synchronize()
    og = oracle.geom(N, F, T)
    src_np = base[..., :d].numpy()
    dst_np = dst.view(idt).cpu().numpy()
    back_np = back.view(idt).cpu().numpy()
    all_np = allp.view(idt).cpu().numpy()
    m = modes.cpu().numpy().reshape(B, H)
    for b in range(B):
        for h in range(H):
            want = oracle.permute_rows(og, np.ascontiguousarray(src_np[b, h]))
            assert np.array_equal(all_np[b, h], want)
            if m[b, h] == svg.TEMPORAL:
                assert np.array_equal(dst_np[b, h], want)
                assert np.array_equal(back_np[b, h], src_np[b, h])
            else:  # untouched
                assert np.all(dst_np[b, h] == 7)
                assert np.all(back_np[b, h] == 0)


@pytest.mark.parametrize("N,F,T,a1,a2,W,St,BM,BN", [
    (5, 37, 3, 2, 5, 40, 100, 128, 64), (33, 60, 0, 2, 7, 60, 512, 128, 64), (4, 64, 0, 1, 8, 64, 16, 64, 64),
    (13, 50, 256, 3, 11, 25, 70, 128, 64), (3, 31, 17, 1, 40, 5, 1, 32, 16)])
def test_build_blocks_bit_exact(N, F, T, a1, a2, W, St, BM, BN):
    H = 6
    g = svg.Geom(B=2, H=H, d=128, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    L = g.L
    nq, nk = -(-L // BM), -(-L // BN)
    modes_np = np.array(MODES6 + MODES6[::-1], dtype=np.int32)
    modes = torch.from_numpy(modes_np).cuda()
    ranges = torch.empty(2 * H * nq * 4, dtype=torch.int32, device="cuda")
    order = torch.empty(2 * H, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes, BM, BN, ranges, order)
    torch.cuda.synchronize()
    r = ranges.cpu().numpy().reshape(2 * H, nq * 4)
    og = ogeom(g)
    work = []
    for bh in range(2 * H):
        got = block_bitmap_from_ranges(r[bh], nq, nk)
        want = oracle.blocks(og, int(modes_np[bh]), BM, BN, brute=L <= 400)
        assert np.array_equal(got, want), (bh, modes_np[bh])
        work.append(int(want.sum()))
    assert np.array_equal(order.cpu().numpy(), oracle.head_order(np.array(work)))


def run_attention(g, q, k, v, modes_np, out_dtype, virtual):
    """Tile lists + layout transformation + attention.  virtual: True (index
    map only), False (token-major copies of Q, K, V and O, O permuted back) or
    "kv" (copies of K and V only, Q and O through the index map: the layer's
    explicit path)."""
    din = svg.BF16 if q.dtype == torch.bfloat16 else svg.F32
    BM, BN = svg.svg_tile_config(din, g.d)
    BH = g.B * g.H
    nq = -(-g.L // BM)
    modes = torch.from_numpy(np.asarray(modes_np, dtype=np.int32)).cuda()
    ranges = torch.empty(BH * nq * 4, dtype=torch.int32, device="cuda")
    order = torch.empty(BH, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes, BM, BN, ranges, order)
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    if virtual is True:
        svg.svg_sparse_attention(g, q, k, v, o, modes, ranges, order, flags=svg.VIRTUAL_PERMUTE)
    elif virtual == "kv":
        kp, vp = (torch.empty_like(t) for t in (k, v))
        for s_, d_ in ((k, kp), (v, vp)):
            svg.svg_layout_permute(g, s_, d_, modes=modes)
        svg.svg_sparse_attention(g, q, k, v, o, modes, ranges, order, kp=kp, vp=vp)
    else:
        qp, kp, vp = (torch.empty_like(t) for t in (q, k, v))
        for s_, d_ in ((q, qp), (k, kp), (v, vp)):
            svg.svg_layout_permute(g, s_, d_, modes=modes)
        op = torch.empty(q.shape, dtype=out_dtype, device="cuda")
        svg.svg_sparse_attention(g, q, k, v, o, modes, ranges, order, qp=qp, kp=kp, vp=vp, op=op)
        svg.svg_layout_permute(g, op, o, modes=modes, inverse=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


ATT_CASES = [
    # dtype, N, F, T, d, a1, a2, window, stripe
    ("bf16", 5, 100, 0, 128, 2, 12, 100, 130),
    ("bf16", 3, 77, 13, 64, 1, 9, 30, 64),
    ("bf16", 9, 40, 5, 128, 3, 6, 50, 70),
    ("f32", 4, 64, 0, 64, 1, 8, 64, 40),
    ("f32", 3, 50, 7, 128, 2, 5, 20, 33),
]


@pytest.mark.parametrize("case", ATT_CASES)
@pytest.mark.parametrize("virtual", [False, True, "kv"])
def test_attention_all_modes(case, virtual):
    dt, N, F, T, d, a1, a2, W, St = case
    H = 6
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    kinds = [planted_kind(m) for m in MODES6]
    inp = S.small_config(N, F, T, H, d, a1, a2, kinds, seed=N + F + d, dtype=dt, window=W, stripe=St)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v = (to_device(inp[n][None], tdt) for n in "qkv")
    outs = [tdt] if dt == "f32" else [torch.bfloat16, torch.float32]
    og = ogeom(g)
    rows = np.arange(g.L)
    for od in outs:
        got = run_attention(g, q, k, v, MODES6, od, virtual)
        for h, mode in enumerate(MODES6):
            ref = oracle.attention_rows(og, mode, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows)
            check_close(got[0, h], ref, dt, what=f"mode {mode} out {od}")


def test_virtual_equals_explicit_and_deterministic():
    N, F, T, d = 6, 90, 10, 128
    g = svg.Geom(B=1, H=6, d=d, N=N, F=F, T=T, a1=2, a2=10, window=45, stripe=100)
    kinds = [planted_kind(m) for m in MODES6]
    inp = S.small_config(N, F, T, 6, d, 2, 10, kinds, seed=77, window=45, stripe=100)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    a = run_attention(g, q, k, v, MODES6, torch.bfloat16, False)
    b = run_attention(g, q, k, v, MODES6, torch.bfloat16, True)
    c = run_attention(g, q, k, v, MODES6, torch.bfloat16, True)
    e = run_attention(g, q, k, v, MODES6, torch.bfloat16, "kv")
    assert np.array_equal(a, b)
    assert np.array_equal(b, c)
    assert np.array_equal(a, e)


@pytest.mark.parametrize("N,F,T", [(64, 3, 0), (65, 2, 7), (100, 2, 5), (130, 1, 3), (7, 40, 70)])
def test_index_map_frame_counts(N, F, T):
    """Temporal heads through the index map (read incrementally from tile to
    tile at d 128: a frame wrap on every tile, exactly one, or one every few
    tiles, and ranges that start in the text prefix) give the same bits as
    the token-major copies, and the oracle's outputs."""
    d, a1, a2 = 128, 2, 3
    g = svg.Geom(B=1, H=6, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=33, stripe=40)
    kinds = [planted_kind(m) for m in MODES6]
    inp = S.small_config(N, F, T, 6, d, a1, a2, kinds, seed=N * 7 + F + T, window=33, stripe=40)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    a = run_attention(g, q, k, v, MODES6, torch.bfloat16, True)
    b = run_attention(g, q, k, v, MODES6, torch.bfloat16, "kv")
    assert np.array_equal(a, b)
    og = ogeom(g)
    rows = np.arange(g.L)
    for h, mode in enumerate(MODES6):
        ref = oracle.attention_rows(og, mode, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows)
        check_close(a[0, h], ref, "bf16", what=f"mode {mode} N {N}")


@pytest.mark.parametrize("dt,N,F,T,d,a1,a2", [
    ("bf16", 6, 96, 0, 128, 2, 12), ("bf16", 5, 120, 20, 64, 1, 20), ("f32", 4, 64, 0, 64, 1, 8),
    ("bf16", 4, 50, 9, 128, 2, 7)])
def test_profile_labels_bit_exact(dt, N, F, T, d, a1, a2):
    kinds = [S.SPATIAL, S.TEMPORAL, S.UNSTRUCTURED, S.TEMPORAL, S.SPATIAL, S.UNSTRUCTURED]
    H = len(kinds)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2)
    inp = S.small_config(N, F, T, H, d, a1, a2, kinds, seed=5 * N + d, dtype=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v = (to_device(inp[n][None], tdt) for n in "qkv")
    rows_np = S.sample_rows(N, F, T, 0.15, 3)
    rows = torch.from_numpy(rows_np).cuda()
    labels = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 3, dtype=torch.float32, device="cuda")
    din = svg.BF16 if dt == "bf16" else svg.F32
    ws = svg.alloc_workspace(g, din, rows.numel(), svg.VIRTUAL_PERMUTE)
    svg.svg_profile_heads(g, q, k, v, rows, labels, stats, ws)
    torch.cuda.synchronize()
    lab = labels.cpu().numpy()
    st = stats.cpu().numpy().reshape(H, 3)
    og = ogeom(g)
    for h in range(H):
        want, ref = oracle.profile_head(og, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows_np)
        assert lab[h] == want, (h, lab[h], want, st[h], ref)
        # statistics: relative errors to 2 % (absolute floor 1e-4 for near-zero errors)
        np.testing.assert_allclose(st[h], ref, rtol=2e-2, atol=1e-4)


@pytest.mark.parametrize("d,seed", [(64, 11), (128, 12)])
def test_profile_on_library_sampled_rows(d, seed):
    """Row sampling and profiling through the library: svg_sample_rows draws
    1 % of the video rows (fresh rows for a new seed), svg_profile_heads
    labels the heads on them, equal to the oracle's labels on the same rows."""
    N, F, T, a1, a2 = 8, 400, 16, 2, 40
    kinds = [S.SPATIAL, S.TEMPORAL, S.SPATIAL, S.TEMPORAL]
    H = len(kinds)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2)
    inp = S.small_config(N, F, T, H, d, a1, a2, kinds, seed=seed)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    count = -(-N * F // 100)
    rows_np = svg.svg_sample_rows(g, count, seed)
    assert not np.array_equal(rows_np, svg.svg_sample_rows(g, count, seed + 1))
    rows = torch.from_numpy(rows_np).cuda()
    labels = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 3, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows.numel(), svg.VIRTUAL_PERMUTE)
    print(f"\n[profile on library rows d={d} rows={count}]", flush=True)
    svg.svg_profile_heads(g, q, k, v, rows, labels, stats, ws)
    torch.cuda.synchronize()
    lab, st = labels.cpu().numpy(), stats.cpu().numpy().reshape(H, 3)
    og = ogeom(g)
    for h in range(H):
        want, ref = oracle.profile_head(og, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows_np)
        assert lab[h] == want, (h, lab[h], want, st[h], ref)
        np.testing.assert_allclose(st[h], ref, rtol=2e-2, atol=1e-4)


LAYOUT_CASES = [
    # B, H, N, F, T, d, a1, a2, window, stripe, modes (B*H of them)
    (2, 3, 4, 50, 5, 128, 1, 6, 40, 60, [svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.WINDOW, svg.STRIPE, svg.SKIP]),
    (1, 2, 1, 200, 0, 64, 1, 30, 50, 64, [svg.SPATIAL, svg.TEMPORAL]),              # one frame
    (1, 2, 150, 1, 3, 128, 4, 1, 9, 20, [svg.SPATIAL, svg.TEMPORAL]),               # one token per frame
    (1, 3, 1, 7, 2, 64, 1, 2, 3, 4, [svg.SPATIAL, svg.TEMPORAL, svg.FULL]),         # shorter than a tile
    (2, 2, 5, 30, 4, 128, 5, 30, 200, 500, [svg.SPATIAL, svg.TEMPORAL, svg.WINDOW, svg.STRIPE]),  # bands wider
]


@pytest.mark.parametrize("case", LAYOUT_CASES)
@pytest.mark.parametrize("virtual", [False, True, "kv"])
def test_attention_strided_batched_and_degenerate(case, virtual):
    """B = 2 with Q, K, V, O as [B, L, H, d] memory viewed as [B, H, L, d]
    (token-interleaved heads), and degenerate geometries: a single frame, one
    token per frame, fewer tokens than one tile, bands wider than the video."""
    B, H, N, F, T, d, a1, a2, W, St, modes = case
    g = svg.Geom(B=B, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    L = g.L
    kinds = [planted_kind(m) for m in modes]
    inp = S.small_config(N, F, T, B * H, d, a1, a2, kinds, seed=B * 100 + N + F, window=W, stripe=St)
    print(f"\n[strided/degenerate B={B} H={H} N={N} F={F} T={T} d={d} virtual={virtual}]", flush=True)

    def interleaved(a, dtype):  # [B*H, L, d] -> [B, L, H, d] memory, viewed [B, H, L, d]
        t = torch.from_numpy(np.ascontiguousarray(a.reshape(B, H, L, d).transpose(0, 2, 1, 3))).to(dtype).cuda()
        return t.permute(0, 2, 1, 3)

    q, k, v = (interleaved(inp[n], torch.bfloat16) for n in "qkv")
    assert q.stride() == (L * H * d, d, H * d, 1)
    BM, BN = svg.svg_tile_config(svg.BF16, d)
    nq = -(-L // BM)
    modes_t = torch.tensor(modes, dtype=torch.int32, device="cuda")
    ranges = torch.empty(B * H * nq * 4, dtype=torch.int32, device="cuda")
    order = torch.empty(B * H, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes_t, BM, BN, ranges, order)
    o = interleaved(np.full((B * H, L, d), np.nan, dtype=np.float32), torch.bfloat16)
    if virtual is True:
        svg.svg_sparse_attention(g, q, k, v, o, modes_t, ranges, order, flags=svg.VIRTUAL_PERMUTE)
    elif virtual == "kv":
        kp, vp = (torch.empty((B, H, L, d), dtype=torch.bfloat16, device="cuda") for _ in range(2))
        for s_, d_ in ((k, kp), (v, vp)):
            svg.svg_layout_permute(g, s_, d_, modes=modes_t)
        svg.svg_sparse_attention(g, q, k, v, o, modes_t, ranges, order, kp=kp, vp=vp)
    else:
        qp, kp, vp = (torch.empty((B, H, L, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
        for s_, d_ in ((q, qp), (k, kp), (v, vp)):
            svg.svg_layout_permute(g, s_, d_, modes=modes_t)
        op = torch.empty((B, H, L, d), dtype=torch.bfloat16, device="cuda")
        svg.svg_sparse_attention(g, q, k, v, o, modes_t, ranges, order, qp=qp, kp=kp, vp=vp, op=op)
        svg.svg_layout_permute(g, op, o, modes=modes_t, inverse=True)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().reshape(B * H, L, d)
    og = ogeom(g)
    rows = np.arange(L)
    for bh, mode in enumerate(modes):
        ref = oracle.attention_rows(og, mode, inp["q"][bh], inp["k"][bh], inp["v"][bh], scale_of(g), rows)
        check_close(got[bh], ref, "bf16", what=f"head {bh} mode {mode}")


@pytest.mark.parametrize("n_rows_frac,seed", [(None, 1), (0.2, 2)])
def test_profile_strided_batched(n_rows_frac, seed):
    """Profiling with B = 2 on token-interleaved [B, L, H, d] memory, once with a
    single sampled row (the smallest sample) and once with 20 % of the rows:
    labels bit-exact, statistics as in the contiguous test."""
    B, H, N, F, T, d, a1, a2 = 2, 3, 5, 60, 6, 128, 2, 9
    kinds = [S.SPATIAL, S.TEMPORAL, S.UNSTRUCTURED, S.TEMPORAL, S.SPATIAL, S.SPATIAL]
    g = svg.Geom(B=B, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2)
    L = g.L
    inp = S.small_config(N, F, T, B * H, d, a1, a2, kinds, seed=40 + seed)
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n].reshape(B, H, L, d).transpose(0, 2, 1, 3)))
         .to(torch.bfloat16).cuda().permute(0, 2, 1, 3) for n in "qkv"}
    rows_np = np.array([T + 77], dtype=np.int32) if n_rows_frac is None else S.sample_rows(N, F, T, n_rows_frac, seed)
    rows = torch.from_numpy(rows_np).cuda()
    labels = torch.empty(B * H, dtype=torch.int32, device="cuda")
    stats = torch.empty(B * H * 3, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows.numel(), svg.VIRTUAL_PERMUTE)
    print(f"\n[profile strided B={B} rows={rows_np.size}]", flush=True)
    svg.svg_profile_heads(g, t["q"], t["k"], t["v"], rows, labels, stats, ws)
    torch.cuda.synchronize()
    lab = labels.cpu().numpy()
    st = stats.cpu().numpy().reshape(B * H, 3)
    og = ogeom(g)
    for bh in range(B * H):
        want, ref = oracle.profile_head(og, inp["q"][bh], inp["k"][bh], inp["v"][bh], scale_of(g), rows_np)
        assert lab[bh] == want, (bh, lab[bh], want, st[bh], ref)
        np.testing.assert_allclose(st[bh], ref, rtol=2e-2, atol=1e-4)


def test_profile_more_rows_than_lds_order():
    """More sampled rows (about 8900) than the position-order kernel stages in
    LDS (8192): the temporal sweep then takes its row order from per-frame
    binary searches in global memory.  Labels bit-exact, statistics as above."""
    N, F, T, d, a1, a2 = 3, 3500, 0, 64, 1, 40
    kinds = [S.TEMPORAL, S.SPATIAL, S.UNSTRUCTURED]
    H = len(kinds)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2)
    inp = S.small_config(N, F, T, H, d, a1, a2, kinds, seed=61)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    rows_np = S.sample_rows(N, F, T, 0.85, 9)
    assert rows_np.size > 8192
    rows = torch.from_numpy(rows_np).cuda()
    labels = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 3, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows.numel(), svg.VIRTUAL_PERMUTE)
    print(f"\n[profile rows={rows_np.size}]", flush=True)
    svg.svg_profile_heads(g, q, k, v, rows, labels, stats, ws)
    torch.cuda.synchronize()
    lab = labels.cpu().numpy()
    st = stats.cpu().numpy().reshape(H, 3)
    og = ogeom(g)
    for h in range(H):
        want, ref = oracle.profile_head(og, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows_np)
        assert lab[h] == want, (h, lab[h], want, st[h], ref)
        np.testing.assert_allclose(st[h], ref, rtol=2e-2, atol=1e-4)
