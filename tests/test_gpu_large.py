"""Tensors of more than 2^31 elements: 20 heads x 2^20 tokens x d 128 per
Q, K, V, O (5.4 GB each in bf16).  Heads 16..19 start past 2^31 elements,
so every kernel of the layer (tile lists, layout transformation, attention,
inverse transformation, profiling sweeps and merge) must address them with
64-bit offsets.  Sampled output rows of those heads against the oracle, and
the profiling statistics of the last head.  Inputs: N(0, 1) from a seeded
torch generator on the device, one head at a time, rounded to bf16."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_video_svg_amd as svg
from helpers import check_close, ogeom, scale_of

pytestmark = pytest.mark.gpu

N, F, H, d = 512, 2048, 20, 128
L = N * F  # 2^20
# cheap modes everywhere; the heads past 2^31 elements take one of each
# sparse mode that reads keys
MODES = [svg.SPATIAL, svg.TEMPORAL, svg.WINDOW, svg.STRIPE, svg.SKIP] * 3 + [svg.SKIP] + \
        [svg.SPATIAL, svg.TEMPORAL, svg.WINDOW, svg.STRIPE]
FAR = list(range(16, 20))


def _inputs(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for _ in range(3):
        t = torch.empty((1, H, L, d), dtype=torch.bfloat16, device="cuda")
        for h in range(H):
            t[0, h] = torch.randn((L, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        out.append(t)
    return out


def test_layer_past_2pow31_elements():
    assert H * L * d > 2 ** 31 and 16 * L * d >= 2 ** 31
    geom = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=0, a1=1, a2=2, window=1024, stripe=512)
    print(f"\n[large layer H={H} L={L} d={d}: {H * L * d} elements per tensor]", flush=True)
    q, k, v = _inputs(2024)
    o = torch.empty_like(q)
    modes = torch.tensor(MODES, dtype=torch.int32, device="cuda")
    ws = svg.alloc_workspace(geom, svg.BF16, 0, 0)
    svg.svg_layer_forward(geom, q, k, v, o, ws, modes_in=modes)
    torch.cuda.synchronize()
    del ws
    og = ogeom(geom)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, F - 1, F, L - F, L - 1], rng.choice(L, 40, replace=False)]))
    for h in FAR:
        qh, kh, vh = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        want = oracle.attention_rows(og, MODES[h], qh, kh, vh, scale_of(geom), rows)
        got = o[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy()
        check_close(got, want, "bf16", what=f"head {h} mode {MODES[h]}")

    # profiling on 64 sampled rows of every head; the last head's statistics
    rows_p = np.sort(rng.choice(L, 64, replace=False)).astype(np.int32)
    labels = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 3, dtype=torch.float32, device="cuda")
    wsp = svg.alloc_workspace(geom, svg.BF16, rows_p.size, svg.VIRTUAL_PERMUTE)
    svg.svg_profile_heads(geom, q, k, v, torch.from_numpy(rows_p).cuda(), labels, stats, wsp)
    torch.cuda.synchronize()
    h = H - 1
    qh, kh, vh = (t[0, h].float().cpu().numpy() for t in (q, k, v))
    want_label, want_stats = oracle.profile_head(og, qh, kh, vh, scale_of(geom), rows_p)
    assert int(labels[h]) == want_label
    np.testing.assert_allclose(stats.cpu().numpy().reshape(H, 3)[h], want_stats, rtol=2e-2, atol=1e-4)


def test_fp8_layer_past_2pow31_elements():
    """The same layer with FP8 scores and FP8 P.V: the E4M3 codes of Q, K
    and V (2.7 GB each, one byte per element) and their scales are indexed
    past 2^31 bytes.  Every step is per head (Q row and K tile scales, one V
    scale per head, per-row softmax state), so each far head's output must be
    bit-identical to the same head run alone, at small offsets (that run's
    arithmetic is held to the oracle by tests/test_gpu_fp8.py)."""
    geom = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=0, a1=1, a2=2, window=1024, stripe=512)
    print(f"\n[large fp8 layer H={H} L={L} d={d}]", flush=True)
    q, k, v = _inputs(4048)
    o = torch.empty_like(q)
    modes = torch.tensor(MODES, dtype=torch.int32, device="cuda")
    flags = svg.FP8_SCORES | svg.FP8_PV
    ws = svg.alloc_workspace(geom, svg.BF16, 0, flags)
    svg.svg_layer_forward(geom, q, k, v, o, ws, modes_in=modes, flags=flags)
    torch.cuda.synchronize()
    del ws
    g1 = svg.Geom(B=1, H=1, d=d, N=N, F=F, T=0, a1=1, a2=2, window=1024, stripe=512)
    ws1 = svg.alloc_workspace(g1, svg.BF16, 0, flags)
    for h in FAR:
        q1, k1, v1 = (t[:, h:h + 1].contiguous() for t in (q, k, v))
        o1 = torch.empty_like(q1)
        svg.svg_layer_forward(g1, q1, k1, v1, o1, ws1, modes_in=modes[h:h + 1].contiguous(), flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(o[:, h:h + 1], o1), f"head {h} mode {MODES[h]}: far result differs from the head alone"
        assert bool(torch.isfinite(o1.float()).all())


def test_svg2_past_2pow31_elements():
    """SVG2 on the same tensors (k-means of Q and K with the default
    initialisation, 256 clusters each, 2 iterations, p = 0.05): its
    permutations, gathered K / V copies and segment tables address heads past
    2^31 elements.  Every step is per head (fixed-order sums), so each far
    head's output, centroids and selection must be bit-identical to the same
    head run alone (whose arithmetic tests/test_gpu_svg2.py holds to the
    oracle)."""
    geom = svg.Geom(B=1, H=H, d=d, N=N, F=F)
    prm = svg.Svg2Params(256, 256, 2, 0.05)
    print(f"\n[large svg2 H={H} L={L} d={d}]", flush=True)
    q, k, v = _inputs(8096)

    def run(g, q, k, v):
        BH = g.B * g.H
        o = torch.empty_like(q)
        mq = torch.empty(BH * prm.C_q * d, dtype=torch.float32, device="cuda")
        mk = torch.empty(BH * prm.C_k * d, dtype=torch.float32, device="cuda")
        sel = torch.empty(BH * prm.C_q * prm.C_k, dtype=torch.uint8, device="cuda")
        ws = torch.empty(svg.svg2_workspace_bytes(g, prm), dtype=torch.uint8, device="cuda")
        svg.svg2_forward(g, prm, q, k, v, o, mq, mk, ws, sel=sel)
        torch.cuda.synchronize()
        return o, mq.view(BH, -1), mk.view(BH, -1), sel.view(BH, -1)

    o, mq, mk, sel = run(geom, q, k, v)
    g1 = svg.Geom(B=1, H=1, d=d, N=N, F=F)
    for h in FAR:
        o1, mq1, mk1, sel1 = run(g1, *(t[:, h:h + 1].contiguous() for t in (q, k, v)))
        assert torch.equal(mq[h], mq1[0]) and torch.equal(mk[h], mk1[0]), f"head {h}: centroids differ"
        assert torch.equal(sel[h], sel1[0]), f"head {h}: selection differs"
        assert torch.equal(o[:, h:h + 1], o1), f"head {h}: output differs from the head alone"
        assert int(sel1.sum()) > 0 and bool(torch.isfinite(o1.float()).all())
