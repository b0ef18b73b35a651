"""GPU parity of the FP8-score path (marked gpu).

svg_quantize_qk against the oracle's FP8 mode (oracle/fp8.py): E4M3 codes and
power-of-two scales bit-exact, Q per natural row, K per 64-row tile of the
head's working layout (token-major for TEMPORAL heads).
svg_sparse_attention_fp8 (and svg_layer_forward with SVG_FLAG_FP8_SCORES)
against the oracle's masked attention on the dequantised Q and K with the
same V: the bf16 bars (max-abs 2e-2, RMS 2e-3), since the products of E4M3
values are exact in the fp32 accumulators and P, V stay bf16 as in the bf16
kernel."""
import numpy as np
import pytest

import oracle
import sparse_attention_video_svg_amd as svg
import svg_synth as S
from helpers import check_close, ogeom, scale_of, to_device
from oracle import fp8

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MODES6 = [svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.SKIP, svg.WINDOW, svg.STRIPE]
PLANT = {svg.SPATIAL: S.SPATIAL, svg.TEMPORAL: S.TEMPORAL, svg.FULL: S.FULL, svg.SKIP: S.FULL,
         svg.WINDOW: S.WINDOW, svg.STRIPE: S.STRIPE}


def quantize_on_gpu(g, q, k, modes_t):
    BH, L, d = g.B * g.H, g.L, g.d
    nkt = -(-L // 64)
    q8 = torch.empty(BH * L * d, dtype=torch.uint8, device="cuda")
    k8 = torch.empty_like(q8)
    sq = torch.empty(BH * L, dtype=torch.float32, device="cuda")
    sk = torch.empty(BH * nkt, dtype=torch.float32, device="cuda")
    svg.svg_quantize_qk(g, q, k, modes_t, q8, sq, k8, sk)
    return q8, sq, k8, sk


def oracle_quant(g, mode, q, k):
    """(q codes, q scales, k codes in working order, k tile scales, dequantised
    q and k in natural order) of one head."""
    og = ogeom(g)
    cq, sq = fp8.quantize_rows(q)
    kw = oracle.permute_rows(og, k) if mode == svg.TEMPORAL else k
    ck, sk = fp8.quantize_tiles(kw)
    kd = fp8.dequant_tiles(ck, sk)
    if mode == svg.TEMPORAL:
        kd = oracle.permute_rows(og, np.ascontiguousarray(kd), inverse=True)
    return cq, sq, ck, sk, fp8.dequant_rows(cq, sq).astype(np.float32), kd.astype(np.float32)


CASES = [(5, 100, 0, 128, 2, 12, 100, 130), (3, 77, 13, 64, 1, 9, 30, 64), (9, 40, 5, 128, 3, 6, 50, 70)]


@pytest.mark.parametrize("N,F,T,d,a1,a2,W,St", CASES)
def test_quantisation_bit_exact(N, F, T, d, a1, a2, W, St):
    H = len(MODES6)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    inp = S.small_config(N, F, T, H, d, a1, a2, [PLANT[m] for m in MODES6], seed=N * F + d, window=W, stripe=St)
    inp["q"][2, 3] = 0.0  # an all-zero row: scale 1, codes 0
    q, k = (to_device(inp[n][None], torch.bfloat16) for n in "qk")
    modes_t = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    print(f"\n[fp8 quantisation N={N} F={F} T={T} d={d}]", flush=True)
    q8, sq, k8, sk = (t.cpu().numpy() for t in quantize_on_gpu(g, q, k, modes_t))
    torch.cuda.synchronize()
    L, nkt = g.L, -(-g.L // 64)
    for h, mode in enumerate(MODES6):
        cq, sq_o, ck, sk_o, _, _ = oracle_quant(g, mode, inp["q"][h], inp["k"][h])
        assert np.array_equal(q8[h * L * d:(h + 1) * L * d].reshape(L, d), cq), f"q codes head {h}"
        assert np.array_equal(sq[h * L:(h + 1) * L], sq_o.astype(np.float32)), f"q scales head {h}"
        assert np.array_equal(k8[h * L * d:(h + 1) * L * d].reshape(L, d), ck), f"k codes head {h}"
        assert np.array_equal(sk[h * nkt:(h + 1) * nkt], sk_o.astype(np.float32)), f"k scales head {h}"


@pytest.mark.parametrize("N,F,T,d,a1,a2,W,St", CASES)
def test_fp8_attention_all_modes(N, F, T, d, a1, a2, W, St):
    H = len(MODES6)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    inp = S.small_config(N, F, T, H, d, a1, a2, [PLANT[m] for m in MODES6], seed=N + F + d, window=W, stripe=St)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    modes_t = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    print(f"\n[fp8 attention N={N} F={F} T={T} d={d}]", flush=True)
    q8, sq, k8, sk = quantize_on_gpu(g, q, k, modes_t)
    BM, BN = svg.svg_tile_config(svg.BF16, d)
    nQT = -(-g.L // BM)
    ranges = torch.empty(H * nQT * 4, dtype=torch.int32, device="cuda")
    order = torch.empty(H, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes_t, BM, BN, ranges, order)
    og = ogeom(g)
    rows = np.arange(g.L)
    for od in (torch.bfloat16, torch.float32):
        o = torch.full(q.shape, float("nan"), dtype=od, device="cuda")
        svg.svg_sparse_attention_fp8(g, q8, sq, k8, sk, v, o, modes_t, ranges, order)
        torch.cuda.synchronize()
        got = o.float().cpu().numpy()
        for h, mode in enumerate(MODES6):
            _, _, _, _, qd, kd = oracle_quant(g, mode, inp["q"][h], inp["k"][h])
            ref = oracle.attention_rows(og, mode, qd, kd, inp["v"][h], scale_of(g), rows)
            check_close(got[0, h], ref, "bf16", what=f"fp8 mode {mode} out {od}")


@pytest.mark.timeout(900)
def test_fp8_layer_hunyuanvideo_shape():
    """The whole layer with fp8 scores on the HunyuanVideo-shaped workload
    (profiling, tile lists, quantisation, attention): labels as the planted
    types, sampled rows of two heads against the oracle on dequantised Q, K."""
    c = S.CONFIGS[2]
    heads = [0, 1]
    inp = S.make_inputs(2, call=0)
    g = svg.Geom(B=1, H=c["H"], d=c["d"], N=c["N"], F=c["F"], T=c["T"], a1=c["a1"], a2=c["a2"], window=c["F"],
                 stripe=512)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    rows = torch.from_numpy(inp["rows"]).cuda()
    ws = svg.alloc_workspace(g, svg.BF16, rows.numel(), svg.FP8_SCORES)
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    labels = torch.full((g.H,), -1, dtype=torch.int32, device="cuda")
    stats = torch.zeros(g.H * 3, dtype=torch.float32, device="cuda")
    print("\n[fp8 layer hunyuanvideo shape]", flush=True)
    svg.svg_layer_forward(g, q, k, v, o, ws, rows=rows, labels_out=labels, stats_out=stats, flags=svg.FP8_SCORES)
    torch.cuda.synchronize()
    lab = labels.cpu().numpy()
    assert np.array_equal(lab, inp["kinds"])
    og = ogeom(g)
    rng = np.random.default_rng(9)
    check_rows = np.unique(np.concatenate([[0, g.L - 1], rng.choice(g.L, 40, replace=False)]))
    got = o[0].float().cpu().numpy()
    for h in heads:
        _, _, _, _, qd, kd = oracle_quant(g, int(lab[h]), inp["q"][h], inp["k"][h])
        ref = oracle.attention_rows(og, int(lab[h]), qd, kd, inp["v"][h], scale_of(g), check_rows)
        check_close(got[h][check_rows], ref, "bf16", what=f"fp8 layer head {h}")
