"""GPU parity of the SVG2 path (svg2_kmeans, svg2_forward) against the
oracle's SVG2 mode (oracle/svg2.py), marked gpu.

Where the oracle's decisions have clear margins (k-means started from the
planted group centres, so every token is far nearer one centroid than any
other), labels, the cluster order and the cluster starts are bit-exact,
centroids within 1e-4 relative (fp32 sums against fp64), the selection is
bit-exact except where the oracle's running mass sits within 1e-4 of p, and
the outputs are within the bf16 bars against the oracle's attention on the
oracle's selection.  From the strided initialisation (where clusters can
split a group and many tokens sit near two centroids) the GPU's own result
is checked for validity: centroids are the means of its labels, each label
is a nearest centroid up to fp32 rounding, the order is the stable sort."""
import math

import numpy as np
import pytest

import sparse_attention_video_svg_amd as svg
import svg_synth as S
from helpers import check_close, to_device
from oracle import svg2 as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def geom(N, F, T, H, d, B=1):
    return svg.Geom(B=B, H=H, d=d, N=N, F=F, T=T)


def run_kmeans(g, x_np, C, iters, init=None):
    BH, L, d = g.B * g.H, g.L, g.d
    x = to_device(x_np.reshape(g.B, g.H, L, d), torch.bfloat16)
    mu = torch.from_numpy(np.ascontiguousarray(init, dtype=np.float32).ravel()).cuda() if init is not None \
        else torch.zeros(BH * C * d, dtype=torch.float32, device="cuda")
    labels = torch.full((BH * L,), -1, dtype=torch.int32, device="cuda")
    perm = torch.full((BH * L,), -1, dtype=torch.int32, device="cuda")
    start = torch.full((BH * (C + 1),), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(svg.svg2_workspace_bytes(g, svg.Svg2Params(C, C, iters, 1.0)), dtype=torch.uint8,
                     device="cuda")
    svg.svg2_kmeans(g, x, C, iters, mu, labels, perm, start, ws,
                    flags=svg.SVG2_INIT_GIVEN if init is not None else 0)
    torch.cuda.synchronize()
    return (mu.cpu().numpy().reshape(BH, C, d), labels.cpu().numpy().reshape(BH, L),
            perm.cpu().numpy().reshape(BH, L), start.cpu().numpy().reshape(BH, C + 1))


@pytest.mark.parametrize("N,F,T,d,G,iters", [(4, 300, 0, 64, 16, 3), (3, 250, 7, 128, 24, 2), (2, 500, 0, 128, 40, 4)])
def test_kmeans_from_planted_centres_bit_exact(N, F, T, d, G, iters):
    H = 3
    g = geom(N, F, T, H, d)
    inp = S.svg2_inputs(N, F, T, H, d, G, seed=N * F + d)
    print(f"\n[svg2 k-means N={N} F={F} T={T} d={d} G={G}]", flush=True)
    for x_name in ("q", "k"):
        mu, lab, perm, start = run_kmeans(g, inp[x_name], G, iters, init=inp["centres"])
        for h in range(H):
            ol, om, on = O.kmeans(inp[x_name][h], G, iters, init=inp["centres"][h])
            op, os_ = O.permutation(ol, G)
            assert np.array_equal(lab[h], ol), f"{x_name} labels head {h}"
            assert np.array_equal(perm[h], op), f"{x_name} perm head {h}"
            assert np.array_equal(start[h], os_), f"{x_name} start head {h}"
            np.testing.assert_allclose(mu[h], om, rtol=1e-4, atol=1e-5)


def test_kmeans_strided_init_is_valid():
    N, F, T, d, H, C = 4, 300, 5, 64, 2, 24
    g = geom(N, F, T, H, d)
    inp = S.svg2_inputs(N, F, T, H, d, 16, seed=3)
    mu, lab, perm, start = run_kmeans(g, inp["q"], C, 3)
    # one more iteration from the final centroids: its labels are the nearest
    # of those centroids, its centroids their means
    mu2, lab2, perm2, start2 = run_kmeans(g, inp["q"], C, 1, init=mu)
    for h in range(H):
        x = inp["q"][h].astype(np.float64)
        for l_, p_, s_ in ((lab[h], perm[h], start[h]), (lab2[h], perm2[h], start2[h])):
            counts = np.bincount(l_, minlength=C)
            assert np.array_equal(s_, np.concatenate([[0], np.cumsum(counts)]))
            assert np.array_equal(p_, np.argsort(l_, kind="stable"))
        counts2 = np.bincount(lab2[h], minlength=C)
        for c in range(C):
            if counts2[c]:
                np.testing.assert_allclose(mu2[h, c], x[lab2[h] == c].mean(axis=0), rtol=1e-4, atol=1e-5)
        dist = ((x[:, None, :] - mu[h][None].astype(np.float64)) ** 2).sum(axis=2)
        best = dist.min(axis=1)
        gap = dist[np.arange(x.shape[0]), lab2[h]] - best
        assert np.all(gap <= 1e-4 * best.clip(1e-6)), "labels are nearest centroids up to rounding"


def forward(g, prm, inp, init, out_dtype=torch.bfloat16):
    BH, L, d = g.B * g.H, g.L, g.d
    q, k, v = (to_device(inp[n].reshape(g.B, g.H, L, d), torch.bfloat16) for n in "qkv")
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    mq = torch.from_numpy(np.ascontiguousarray(init, dtype=np.float32).ravel()).cuda()
    mk = mq.clone()
    sel = torch.zeros(BH * prm.C_q * prm.C_k, dtype=torch.uint8, device="cuda")
    ws = torch.empty(svg.svg2_workspace_bytes(g, prm), dtype=torch.uint8, device="cuda")
    svg.svg2_forward(g, prm, q, k, v, o, mq, mk, ws, sel=sel, flags=svg.SVG2_INIT_GIVEN)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy().reshape(BH, L, d), sel.cpu().numpy().reshape(BH, prm.C_q, prm.C_k),
            mq.cpu().numpy().reshape(BH, prm.C_q, d), mk.cpu().numpy().reshape(BH, prm.C_k, d))


def clear_selection_rows(ref, p):
    """Query clusters whose selection boundary is far from p in the oracle."""
    rows = []
    for a in range(ref["P"].shape[0]):
        Pa = ref["P"][a]
        order = sorted(range(Pa.size), key=lambda b: (-Pa[b], b))
        before = np.concatenate([[0.0], np.cumsum(Pa[order])])[:-1]
        if np.all(np.abs(before - p) > 1e-4):
            rows.append(a)
    return rows


@pytest.mark.parametrize("N,F,T,d,G,spread,p,B", [(4, 300, 0, 64, 16, 1.0, 0.9, 1), (3, 250, 7, 128, 24, 1.0, 0.5, 1),
                                                 (4, 200, 0, 128, 16, 0.35, 0.9, 2), (2, 300, 3, 64, 12, 0.3, 0.7, 1)])
def test_forward_against_oracle(N, F, T, d, G, spread, p, B):
    H = 2
    g = geom(N, F, T, H, d, B=B)
    inp = S.svg2_inputs(N, F, T, B * H, d, G, seed=7 * N + d, spread=spread)
    prm = svg.Svg2Params(G, G, 3, p)
    print(f"\n[svg2 forward N={N} F={F} T={T} d={d} G={G} spread={spread} p={p} B={B}]", flush=True)
    out, sel, mq, mk = forward(g, prm, inp, inp["centres"])
    scale = 1.0 / math.sqrt(d)
    n_multi = 0
    for h in range(B * H):
        ref = O.head(inp["q"][h], inp["k"][h], inp["v"][h], G, G, 3, p, scale, init_q=inp["centres"][h],
                     init_k=inp["centres"][h])
        np.testing.assert_allclose(mq[h], ref["mu_q"], rtol=1e-4, atol=1e-5)
        np.testing.assert_allclose(mk[h], ref["mu_k"], rtol=1e-4, atol=1e-5)
        rows_ok = clear_selection_rows(ref, p)
        assert len(rows_ok) >= G // 2
        for a in rows_ok:
            assert np.array_equal(sel[h, a].astype(bool), ref["sel"][a]), (h, a)
        n_multi += int((ref["sel"].sum(axis=1) > 1).sum())
        # outputs against the oracle on the GPU's own selection where it differs
        use_sel = sel[h].astype(bool)
        want = O.attention_rows(inp["q"][h], inp["k"][h], inp["v"][h], ref["labels_q"], ref["labels_k"], use_sel,
                                scale, np.arange(g.L))
        check_close(out[h], want, "bf16", what=f"svg2 head {h}")
    if spread < 0.5:
        assert n_multi > 0  # the low-separation cases select several key clusters somewhere


@pytest.mark.timeout(900)
def test_forward_hunyuanvideo_shape_sampled_rows():
    """The HunyuanVideo-shaped layer (33 x 3600 tokens, d 128), two heads,
    256 groups, k-means from the planted centres, p = 0.9: outputs of 64
    sampled rows per head against the oracle (its attention on the oracle's
    clustering and the GPU's selection)."""
    N, F, T, d, G, H = 33, 3600, 0, 128, 256, 2
    g = geom(N, F, T, H, d)
    inp = S.svg2_inputs(N, F, T, H, d, G, seed=11)
    prm = svg.Svg2Params(G, G, 2, 0.9)
    out, sel, mq, mk = forward(g, prm, inp, inp["centres"])
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(g.L, 64, replace=False))
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        # the oracle's k-means on the full head (numpy, G x L distances per iteration)
        lq, muq, _ = O.kmeans(inp["q"][h], G, 2, init=inp["centres"][h])
        lk, muk, _ = O.kmeans(inp["k"][h], G, 2, init=inp["centres"][h])
        np.testing.assert_allclose(mq[h], muq, rtol=1e-4, atol=1e-5)
        want = O.attention_rows(inp["q"][h], inp["k"][h], inp["v"][h], lq, lk, sel[h].astype(bool), scale, rows)
        check_close(out[h][rows], want, "bf16", what=f"svg2 large head {h}")


def dense_reference(g, inp, h):
    import oracle
    og = oracle.geom(g.N, g.F, g.T, 1, 1, 1, 1)
    return oracle.attention_rows(og, oracle.FULL, inp["q"][h], inp["k"][h], inp["v"][h], 1.0 / math.sqrt(g.d),
                                 np.arange(g.L))


@pytest.mark.parametrize("C,p,od", [(1, 0.3, torch.bfloat16), (12, 1.5, torch.bfloat16), (12, 1.5, torch.float32)])
def test_degenerate_selections_are_dense_attention(C, p, od):
    """One cluster, or p above 1 (every non-empty key cluster selected): the
    step is dense attention over all keys (the oracle's C routine)."""
    N, F, T, d, H = 3, 130, 9, 128, 2
    g = geom(N, F, T, H, d)
    inp = S.svg2_inputs(N, F, T, H, d, 12, seed=21, spread=0.5)
    prm = svg.Svg2Params(C, C, 2, p)
    print(f"\n[svg2 dense limit C={C} p={p} out={od}]", flush=True)
    init = np.stack([O.strided_init(inp["q"][h], C) for h in range(H)]).astype(np.float32)
    out, sel, _, _ = forward(g, prm, inp, init, out_dtype=od)
    for h in range(H):
        counts = np.bincount(O.kmeans(inp["k"][h], C, 2, init=init[h])[0], minlength=C)
        assert np.array_equal(sel[h].astype(bool), np.broadcast_to(counts > 0, (C, C)))
        check_close(out[h], dense_reference(g, inp, h), "bf16", what=f"dense limit head {h}")


def test_one_token_per_cluster():
    """C = L: every token its own cluster (the strided initialisation puts a
    centroid on each token), so the cluster estimate is the exact attention
    weight and top-p picks the heaviest keys of each query."""
    N, F, T, d, H = 2, 40, 0, 64, 2
    g = geom(N, F, T, H, d)
    inp = S.svg2_inputs(N, F, T, H, d, 8, seed=4, spread=0.2)
    L = g.L
    prm = svg.Svg2Params(L, L, 1, 0.9)
    q, k, v = (to_device(inp[n].reshape(1, H, L, d), torch.bfloat16) for n in "qkv")
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    mq = torch.zeros(H * L * d, dtype=torch.float32, device="cuda")
    mk = torch.zeros_like(mq)
    sel = torch.zeros(H * L * L, dtype=torch.uint8, device="cuda")
    ws = torch.empty(svg.svg2_workspace_bytes(g, prm), dtype=torch.uint8, device="cuda")
    print("\n[svg2 one token per cluster]", flush=True)
    svg.svg2_forward(g, prm, q, k, v, o, mq, mk, ws, sel=sel)
    torch.cuda.synchronize()
    out = o.float().cpu().numpy().reshape(H, L, d)
    sel = sel.cpu().numpy().reshape(H, L, L)
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        ref = O.head(inp["q"][h], inp["k"][h], inp["v"][h], L, L, 1, 0.9, scale)
        assert np.array_equal(ref["labels_q"], np.arange(L)) and np.array_equal(ref["labels_k"], np.arange(L))
        rows_ok = clear_selection_rows(ref, 0.9)
        assert len(rows_ok) >= L // 2
        for a in rows_ok:
            assert np.array_equal(sel[h, a].astype(bool), ref["sel"][a]), (h, a)
        want = O.attention_rows(inp["q"][h], inp["k"][h], inp["v"][h], ref["labels_q"], ref["labels_k"],
                                sel[h].astype(bool), scale, np.arange(L))
        check_close(out[h], want, "bf16", what=f"one token per cluster head {h}")


def test_forward_strided_init_consistent():
    """Forward from the strided initialisation: its centroids equal
    svg2_kmeans's (the same deterministic kernels); the selection matches the
    oracle's top-p on those centroids and cluster sizes where the boundary is
    clear; outputs match the oracle's attention on the GPU's own clustering
    and selection."""
    N, F, T, d, H, C = 4, 220, 6, 128, 2, 20
    g = geom(N, F, T, H, d)
    inp = S.svg2_inputs(N, F, T, H, d, 14, seed=8, spread=0.4)
    prm = svg.Svg2Params(C, C, 3, 0.8)
    L = g.L
    q, k, v = (to_device(inp[n].reshape(1, H, L, d), torch.bfloat16) for n in "qkv")
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    mq = torch.zeros(H * C * d, dtype=torch.float32, device="cuda")
    mk = torch.zeros_like(mq)
    sel = torch.zeros(H * C * C, dtype=torch.uint8, device="cuda")
    ws = torch.empty(svg.svg2_workspace_bytes(g, prm), dtype=torch.uint8, device="cuda")
    print("\n[svg2 forward strided init]", flush=True)
    svg.svg2_forward(g, prm, q, k, v, o, mq, mk, ws, sel=sel)
    torch.cuda.synchronize()
    kq = run_kmeans(g, inp["q"], C, 3)
    kk = run_kmeans(g, inp["k"], C, 3)
    assert np.array_equal(mq.cpu().numpy().reshape(H, C, d), kq[0])
    assert np.array_equal(mk.cpu().numpy().reshape(H, C, d), kk[0])
    out = o.float().cpu().numpy().reshape(H, L, d)
    sel = sel.cpu().numpy().reshape(H, C, C)
    scale = 1.0 / math.sqrt(d)
    n_multi = 0
    for h in range(H):
        counts = np.bincount(kk[1][h], minlength=C)
        P = O.cluster_scores(kq[0][h], kk[0][h], counts, scale)
        ref = dict(P=P)
        want_sel = O.top_p(P, counts, 0.8)
        rows_ok = clear_selection_rows(ref, 0.8)
        assert len(rows_ok) >= C // 2
        for a in rows_ok:
            assert np.array_equal(sel[h, a].astype(bool), want_sel[a]), (h, a)
        n_multi += int((want_sel.sum(axis=1) > 1).sum())
        want = O.attention_rows(inp["q"][h], inp["k"][h], inp["v"][h], kq[1][h], kk[1][h], sel[h].astype(bool),
                                scale, np.arange(L))
        check_close(out[h], want, "bf16", what=f"strided forward head {h}")
    assert n_multi > 0


def test_forward_strided_equals_contiguous():
    """Q, K, V, O as token-interleaved [B, L, H, d] memory viewed as
    [B, H, L, d]: every output bit-identical to the contiguous run (only the
    addresses differ), B = 2."""
    N, F, T, d, H, B, G = 3, 120, 5, 128, 2, 2, 10
    g = geom(N, F, T, H, d, B=B)
    L = g.L
    inp = S.svg2_inputs(N, F, T, B * H, d, G, seed=12, spread=0.4)
    prm = svg.Svg2Params(G, G, 2, 0.8)
    print("\n[svg2 strided vs contiguous]", flush=True)
    outs = []
    for interleave in (False, True):
        if interleave:
            q, k, v = (torch.from_numpy(np.ascontiguousarray(inp[n].reshape(B, H, L, d).transpose(0, 2, 1, 3)))
                       .to(torch.bfloat16).cuda().permute(0, 2, 1, 3) for n in "qkv")
            o = torch.full((B, L, H, d), float("nan"), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
        else:
            q, k, v = (to_device(inp[n].reshape(B, H, L, d), torch.bfloat16) for n in "qkv")
            o = torch.full((B, H, L, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        mq = torch.zeros(B * H * G * d, dtype=torch.float32, device="cuda")
        mk = torch.zeros_like(mq)
        sel = torch.zeros(B * H * G * G, dtype=torch.uint8, device="cuda")
        ws = torch.empty(svg.svg2_workspace_bytes(g, prm), dtype=torch.uint8, device="cuda")
        svg.svg2_forward(g, prm, q, k, v, o, mq, mk, ws, sel=sel)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), mq.cpu().numpy(), mk.cpu().numpy(), sel.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
