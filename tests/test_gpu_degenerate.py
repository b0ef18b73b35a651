"""Degenerate geometries at the edges of the tiling: a single token, a single
video token behind one text token, one token past a full key tile, one token
per frame behind a text prefix.  Every mode through the whole layer (bf16 and
FP8 scores + FP8 P.V) and profiling over every video row, against the
oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_video_svg_amd as svg
import svg_synth as S
from helpers import check_close, ogeom, scale_of, to_device

pytestmark = pytest.mark.gpu

MODES6 = [svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.SKIP, svg.WINDOW, svg.STRIPE]
PLANT = {svg.SPATIAL: S.SPATIAL, svg.TEMPORAL: S.TEMPORAL, svg.FULL: S.UNSTRUCTURED, svg.SKIP: S.UNSTRUCTURED,
         svg.WINDOW: S.SPATIAL, svg.STRIPE: S.UNSTRUCTURED}
# N, F, T, d, a1, a2, window, stripe
CASES = [(1, 1, 0, 64, 1, 1, 1, 1), (1, 1, 1, 128, 1, 1, 1, 1), (1, 65, 0, 128, 1, 3, 2, 64),
         (5, 1, 3, 64, 2, 1, 2, 3), (2, 64, 0, 128, 1, 64, 64, 64)]


def _setup(case, seed):
    N, F, T, d, a1, a2, W, St = case
    H = len(MODES6)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    inp = S.small_config(N, F, T, H, d, a1, a2, [PLANT[m] for m in MODES6], seed=seed, window=W, stripe=St)
    return g, inp


@pytest.mark.parametrize("case", CASES)
def test_layer_all_modes(case):
    g, inp = _setup(case, 300 + sum(case))
    print(f"\n[degenerate layer {case} L={g.L}]", flush=True)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    modes = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, 0, 0)
    svg.svg_layer_forward(g, q, k, v, o, ws, modes_in=modes)
    torch.cuda.synchronize()
    got = o[0].float().cpu().numpy()
    og, rows = ogeom(g), np.arange(g.L)
    for h, mode in enumerate(MODES6):
        want = oracle.attention_rows(og, mode, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows)
        check_close(got[h], want, "bf16", what=f"mode {mode}")


@pytest.mark.parametrize("case", CASES)
def test_fp8_layer_all_modes(case):
    from oracle import fp8
    from test_gpu_fp8 import check_fp8_pv_rows, oracle_quant
    g, inp = _setup(case, 400 + sum(case))
    print(f"\n[degenerate fp8 layer {case} L={g.L}]", flush=True)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    modes = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    flags = svg.FP8_SCORES | svg.FP8_PV
    ws = svg.alloc_workspace(g, svg.BF16, 0, flags)
    svg.svg_layer_forward(g, q, k, v, o, ws, modes_in=modes, flags=flags)
    torch.cuda.synchronize()
    got = o[0].float().cpu().numpy()
    og, rows = ogeom(g), np.arange(g.L)
    for h, mode in enumerate(MODES6):
        _, _, _, _, qd, kd = oracle_quant(g, mode, inp["q"][h], inp["k"][h])
        cv, s = fp8.quantize_head(inp["v"][h])
        vd = (fp8.e4m3_decode(cv) * s).astype(np.float32)
        check_fp8_pv_rows(got[h], qd, kd, vd, og, mode, scale_of(g), rows, f"fp8 mode {mode}")


@pytest.mark.parametrize("case", CASES)
def test_profile_every_video_row(case):
    g, inp = _setup(case, 500 + sum(case))
    print(f"\n[degenerate profile {case} L={g.L}]", flush=True)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    rows_np = np.arange(g.T, g.L, dtype=np.int32)
    labels = torch.empty(g.H, dtype=torch.int32, device="cuda")
    stats = torch.empty(g.H * 3, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows_np.size, svg.VIRTUAL_PERMUTE)
    svg.svg_profile_heads(g, q, k, v, torch.from_numpy(rows_np).cuda(), labels, stats, ws)
    torch.cuda.synchronize()
    lab, st = labels.cpu().numpy(), stats.cpu().numpy().reshape(g.H, 3)
    og = ogeom(g)
    for h in range(g.H):
        want, ref = oracle.profile_head(og, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), rows_np)
        np.testing.assert_allclose(st[h], ref, rtol=2e-2, atol=1e-4)
        # the label is compared where both statistics are clear of each other
        # and of the fallback threshold (a tie of two masks that both equal
        # full attention here is decided by rounding on either side)
        rs, rt = ref[0], ref[1]
        if abs(rs - rt) > 0.05 * max(rs, rt) + 1e-3 and abs(min(rs, rt) - 0.05) > 5e-3:
            assert lab[h] == want, (h, lab[h], want, st[h], ref)


@pytest.mark.parametrize("d", [64, 128])
def test_profile_rows_outside_contract(d, monkeypatch):
    """A row list that breaks the contract (rows outside [T, L), repeats, no
    order) is clamped into [T, L) as read: profiling then equals the oracle's
    on the clamped list, row for row, and nothing is read outside q, k, v."""
    monkeypatch.setattr(svg, "DEBUG", False)
    N, F, T, H = 4, 64, 3, 2
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=1, a2=8)
    inp = S.small_config(N, F, T, H, d, 1, 8, [S.SPATIAL, S.TEMPORAL], seed=77 + d)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    rows_np = np.array([g.L + 40, -7, T + 10, T + 10, g.L - 1, T + 130, 0, T + 5, T + 130, 2**31 - 1],
                       dtype=np.int32)
    clamped = np.clip(rows_np.astype(np.int64), T, g.L - 1)
    print(f"\n[profile rows outside the contract d={d} L={g.L}]", flush=True)
    labels = torch.empty(H, dtype=torch.int32, device="cuda")
    stats = torch.empty(H * 3, dtype=torch.float32, device="cuda")
    ws = svg.alloc_workspace(g, svg.BF16, rows_np.size, svg.VIRTUAL_PERMUTE)
    svg.svg_profile_heads(g, q, k, v, torch.from_numpy(rows_np).cuda(), labels, stats, ws)
    torch.cuda.synchronize()
    st = stats.cpu().numpy().reshape(H, 3)
    og = ogeom(g)
    for h in range(H):
        _, ref = oracle.profile_head(og, inp["q"][h], inp["k"][h], inp["v"][h], scale_of(g), clamped)
        np.testing.assert_allclose(st[h], ref, rtol=2e-2, atol=1e-4)
