"""The GPU path against closed forms, with no oracle in between: Q = 0 makes
every score equal (each bf16 weight is exactly 1), so every masked attention
output is the plain mean of V over the row's active keys, and the profiling
statistics follow from those means.  Masks are the pages' definitions
written out here (text keys and rows dense; spatial |i1 - i2| < a1, temporal
|j1 - j2| < a2, window |u1 - u2| < W, stripe u2 < stripe, skip none)."""
import numpy as np
import pytest
import torch

import sparse_attention_video_svg_amd as svg
import svg_synth as S
from helpers import to_device

pytestmark = pytest.mark.gpu

MODES6 = [svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.SKIP, svg.WINDOW, svg.STRIPE]


def active_keys(g, mode, x):
    L, T, F = g.L, g.T, g.F
    if mode == svg.SKIP:
        return np.zeros(0, np.int64)
    x2 = np.arange(L)
    if x < T:
        return x2
    u1, u2 = x - T, x2 - T
    if mode == svg.SPATIAL:
        keep = np.abs(u1 // F - u2 // F) < g.a1
    elif mode == svg.TEMPORAL:
        keep = np.abs(u1 % F - u2 % F) < g.a2
    elif mode == svg.WINDOW:
        keep = np.abs(u1 - u2) < g.window
    elif mode == svg.STRIPE:
        keep = u2 < g.stripe
    else:
        keep = np.ones(L, bool)
    return x2[(x2 < T) | keep]


def bf16_values(shape, rng, shift=0.0):
    a = (rng.standard_normal(shape) + shift).astype(np.float32)
    return S.bf16_to_f32(S.bf16_bits(a)).reshape(shape)


@pytest.mark.parametrize("N,F,T,d,a1,a2,W,St", [(5, 70, 0, 128, 2, 9, 40, 100), (4, 90, 6, 64, 1, 12, 30, 64)])
def test_attention_means_all_modes(N, F, T, d, a1, a2, W, St):
    H = len(MODES6)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    rng = np.random.default_rng(N * F + d)
    v = bf16_values((H, g.L, d), rng, 0.3)
    q, k, vt = (to_device(a[None], torch.bfloat16)
                for a in (np.zeros((H, g.L, d), np.float32), bf16_values((H, g.L, d), rng), v))
    o = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    modes = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, 0, 0)
    print(f"\n[closed form attention N={N} F={F} T={T} d={d}]", flush=True)
    svg.svg_layer_forward(g, q, k, vt, o, ws, modes_in=modes)
    torch.cuda.synchronize()
    got = o[0].cpu().numpy()
    vd = v.astype(np.float64)
    for h, mode in enumerate(MODES6):
        want = np.stack([vd[h][active_keys(g, mode, x)].mean(axis=0) if mode != svg.SKIP else np.zeros(d)
                         for x in range(g.L)])
        # weights are exactly 1: only fp32 summation (about 350 terms) separates the two
        np.testing.assert_allclose(got[h], want, rtol=0, atol=1e-5, err_msg=f"mode {mode}")


@pytest.mark.parametrize("N,F,T,d,a1,a2", [(6, 64, 0, 128, 2, 8), (5, 50, 4, 64, 1, 50)])
def test_profile_statistics_from_means(N, F, T, d, a1, a2):
    H = 2
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2)
    rng = np.random.default_rng(3 * N + F)
    v = bf16_values((H, g.L, d), rng, 0.5)
    q, k, vt = (to_device(a[None], torch.bfloat16)
                for a in (np.zeros((H, g.L, d), np.float32), bf16_values((H, g.L, d), rng), v))
    rows_np = S.sample_rows(N, F, T, 0.3, 7)
    labels = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 3, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows_np.size, svg.VIRTUAL_PERMUTE)
    print(f"\n[closed form profiling N={N} F={F} T={T} d={d}]", flush=True)
    svg.svg_profile_heads(g, q, k, vt, torch.from_numpy(rows_np).cuda(), labels, stats, ws)
    torch.cuda.synchronize()
    st = stats.cpu().numpy().reshape(H, 3)
    lab = labels.cpu().numpy()
    for h in range(H):
        vd = v[h].astype(np.float64)
        full = np.repeat(vd.mean(axis=0)[None], rows_np.size, axis=0)
        sp = np.stack([vd[active_keys(g, svg.SPATIAL, x)].mean(axis=0) for x in rows_np])
        te = np.stack([vd[active_keys(g, svg.TEMPORAL, x)].mean(axis=0) for x in rows_np])
        den = (full ** 2).sum()
        want = np.array([((sp - full) ** 2).sum() / den, ((te - full) ** 2).sum() / den, (full ** 2).mean()])
        np.testing.assert_allclose(st[h], want, rtol=1e-3, atol=1e-7, err_msg=f"head {h}")
        rs, rt = want[0], want[1]
        if abs(rs - rt) > 0.01 * max(rs, rt) and abs(min(rs, rt) - 0.05) > 1e-3:
            assert lab[h] == (svg.FULL if min(rs, rt) >= 0.05 else svg.SPATIAL if rs <= rt else svg.TEMPORAL)


@pytest.mark.parametrize("N,F,T,d,W,St,a2", [(5, 40, 0, 128, 40, 64, 6), (4, 48, 5, 64, 20, 30, 48)])
def test_search_mse_from_means(N, F, T, d, W, St, a2):
    """svg_search_modes with Q = 0: each candidate's MSE against full
    attention over the sampled rows follows from means of V (skip: mean of
    O_full^2), and each loss is MSE + lam * (1 - S) with S from pair counts."""
    H, lam = 2, 0.4
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=2, a2=a2, window=W, stripe=St)
    rng = np.random.default_rng(5 * N + F + d)
    v = bf16_values((H, g.L, d), rng, -0.4)
    q, k, vt = (to_device(a[None], torch.bfloat16)
                for a in (np.zeros((H, g.L, d), np.float32), bf16_values((H, g.L, d), rng), v))
    rows_np = S.sample_rows(N, F, T, 0.25, 3)
    modes = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 8, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows_np.size, svg.MODE_SEARCH)
    print(f"\n[closed form search N={N} F={F} T={T} d={d}]", flush=True)
    svg.svg_search_modes(g, q, k, vt, torch.from_numpy(rows_np).cuda(), modes, stats, ws, lam=lam, eps=10.0)
    torch.cuda.synchronize()
    st = stats.cpu().numpy().reshape(H, 8)
    L = g.L
    sparsity = []
    for c in svg.SEARCH_CANDIDATES:
        nnz = 0 if c == svg.SKIP else sum(active_keys(g, c, x).size for x in range(L))
        sparsity.append(1.0 - nnz / L ** 2)
    for h in range(H):
        vd = v[h].astype(np.float64)
        full = np.repeat(vd.mean(axis=0)[None], rows_np.size, axis=0)
        mse = []
        for c in svg.SEARCH_CANDIDATES:
            out = np.stack([vd[active_keys(g, c, x)].mean(axis=0) if c != svg.SKIP else np.zeros(d)
                            for x in rows_np])
            mse.append(((out - full) ** 2).mean())
        want_loss = np.array(mse) + lam * (1.0 - np.array(sparsity))
        np.testing.assert_allclose(st[h, :4], mse, rtol=1e-3, atol=1e-8, err_msg=f"mse head {h}")
        np.testing.assert_allclose(st[h, 4:], want_loss, rtol=1e-3, atol=1e-8, err_msg=f"loss head {h}")
