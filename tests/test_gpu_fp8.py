"""GPU parity of the FP8-score path (marked gpu).

svg_quantize_qk against the oracle's FP8 mode (oracle/fp8.py): E4M3 codes and
power-of-two scales bit-exact, Q per natural row, K per 64-row tile of the
head's working layout (token-major for TEMPORAL heads).
svg_sparse_attention_fp8 (and svg_layer_forward with SVG_FLAG_FP8_SCORES)
against the oracle's masked attention on the dequantised Q and K with the
same V: the bf16 bars (max-abs 2e-2, RMS 2e-3), since the products of E4M3
values are exact in the fp32 accumulators and P, V stay bf16 as in the bf16
kernel."""
import math

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
    c = S.WORKLOADS[S.HUNYUANVIDEO]
    heads = [0, 1]
    inp = S.make_inputs(S.HUNYUANVIDEO, call=0)
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


# ---------------------------------------------------------------------------
# FP8 P.V (svg_quantize_v, svg_sparse_attention_fp8_pv, SVG_FLAG_FP8_PV):
# V codes and per-head scales bit-exact against the oracle's per-head
# quantisation; outputs against the oracle's exact softmax attention on the
# dequantised Q, K, V, within the analytic bound of the E4M3 weights
# (tests/fp8_bounds.py) plus the bf16 output rounding.

def quantize_v_on_gpu(g, v, modes_t):
    nkt = -(-g.L // 64)
    v8 = torch.empty(g.B * g.H * nkt * g.d * 64, dtype=torch.uint8, device="cuda")
    sv = torch.empty(g.B * g.H, dtype=torch.float32, device="cuda")
    svg.svg_quantize_v(g, v, modes_t, v8, sv)
    return v8, sv


def v8_natural(v8, g, h, mode):
    """Codes of head h back in natural row order ([L, d]) from the documented
    layout, and the codes of the rows beyond L (padding of the last tile)."""
    nkt = -(-g.L // 64)
    tiles = v8.reshape(g.B * g.H, nkt, g.d, 64)[h]
    p = np.arange(64)
    grp, j = p // 32, p % 32
    key = 32 * (j // 16) + 8 * ((j % 16) // 4) + 4 * grp + j % 4
    work = np.zeros((nkt * 64, g.d), dtype=np.uint8)
    for t in range(nkt):
        work[t * 64 + key] = tiles[t].T
    nat = work[:g.L]
    if mode == svg.TEMPORAL:
        nat = oracle.permute_rows(ogeom(g), np.ascontiguousarray(nat), inverse=True)
    return nat, work[g.L:]


def check_fp8_pv_rows(got, qd, kd, vd, og, mode, scale, rows, what):
    """got [len(rows), d] against the exact attention on dequantised inputs,
    element by element within the E4M3-weight bound."""
    from fp8_bounds import fp8_pv_bound
    ref = oracle.attention_rows(og, mode, qd, kd, vd, scale, rows)
    worst = 0.0
    for i, r in enumerate(rows):
        if mode == svg.SKIP:
            assert np.all(got[i] == 0), what
            continue
        iv = oracle.row_intervals(og, oracle.TEMPORAL if mode == svg.TEMPORAL else mode, int(r))
        keys = np.concatenate([np.arange(lo, hi) for lo, hi in iv])
        x = (kd[keys].astype(np.float64) @ qd[r].astype(np.float64)) * scale / math.log(2.0)
        w = np.exp2(x - x.max())
        w /= w.sum()
        b8 = fp8_pv_bound(x, w, vd[keys], ref[i])
        # bf16 output: rounding to 8 significant bits (half an ulp, at most
        # 2^-8 relative) of the kernel's fp32 value, which lies within b8 of
        # the reference
        bound = b8 + 2.0 ** -8 * (np.abs(ref[i]) + b8) + 1e-4
        err = np.abs(got[i].astype(np.float64) - ref[i])
        assert np.all(err <= bound), f"{what}: row {r} err {err.max():.3e} > bound {bound[np.argmax(err - bound)]:.3e}"
        worst = max(worst, float(np.max(err / bound)))
    return worst


@pytest.mark.parametrize("N,F,T,d,a1,a2,W,St", CASES)
def test_quantize_v_bit_exact(N, F, T, d, a1, a2, W, St):
    H = len(MODES6)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    inp = S.small_config(N, F, T, H, d, a1, a2, [PLANT[m] for m in MODES6], seed=N * F + d + 1, window=W, stripe=St)
    inp["v"][4] = 0.0  # an all-zero head: scale 1, codes 0
    v = to_device(inp["v"][None], torch.bfloat16)
    modes_t = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    print(f"\n[fp8 V quantisation N={N} F={F} T={T} d={d}]", flush=True)
    v8, sv = quantize_v_on_gpu(g, v, modes_t)
    torch.cuda.synchronize()
    v8, sv = v8.cpu().numpy(), sv.cpu().numpy()
    for h, mode in enumerate(MODES6):
        codes, s = fp8.quantize_head(inp["v"][h])
        nat, pad = v8_natural(v8, g, h, mode)
        assert sv[h] == np.float32(s), f"scale head {h}"
        assert np.array_equal(nat, codes), f"codes head {h}"
        assert np.all(pad == 0), f"padding head {h}"


@pytest.mark.parametrize("N,F,T,d,a1,a2,W,St", CASES)
def test_fp8_pv_attention_all_modes(N, F, T, d, a1, a2, W, St):
    H = len(MODES6)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=W, stripe=St)
    inp = S.small_config(N, F, T, H, d, a1, a2, [PLANT[m] for m in MODES6], seed=N + F + d + 2, window=W, stripe=St)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    modes_t = torch.tensor(MODES6, dtype=torch.int32, device="cuda")
    print(f"\n[fp8 P.V attention N={N} F={F} T={T} d={d}]", flush=True)
    q8, sq, k8, sk = quantize_on_gpu(g, q, k, modes_t)
    v8, sv = quantize_v_on_gpu(g, v, modes_t)
    BM, BN = svg.svg_tile_config(svg.BF16, d)
    nQT = -(-g.L // BM)
    ranges = torch.empty(H * nQT * 4, dtype=torch.int32, device="cuda")
    order = torch.empty(H, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes_t, BM, BN, ranges, order)
    og = ogeom(g)
    rows = np.arange(g.L)
    for od in (torch.bfloat16, torch.float32):
        o = torch.full(q.shape, float("nan"), dtype=od, device="cuda")
        svg.svg_sparse_attention_fp8_pv(g, q8, sq, k8, sk, v8, sv, o, modes_t, ranges, order)
        torch.cuda.synchronize()
        got = o.float().cpu().numpy()
        for h, mode in enumerate(MODES6):
            _, _, _, _, qd, kd = oracle_quant(g, mode, inp["q"][h], inp["k"][h])
            cv, s = fp8.quantize_head(inp["v"][h])
            vd = (fp8.e4m3_decode(cv) * s).astype(np.float32)
            worst = check_fp8_pv_rows(got[0, h], qd, kd, vd, og, mode, scale_of(g), rows, f"fp8 P.V mode {mode} {od}")
            print(f"  mode {mode} {od}: worst err / bound {worst:.3f}", flush=True)


@pytest.mark.timeout(900)
def test_fp8_pv_layer_hunyuanvideo_shape():
    """The whole layer with FP8 scores and FP8 P.V on the HunyuanVideo-shaped
    workload: labels as the planted types, sampled rows of two heads within
    the E4M3-weight bound of the oracle on dequantised Q, K, V."""
    c = S.WORKLOADS[S.HUNYUANVIDEO]
    inp = S.make_inputs(S.HUNYUANVIDEO, call=0)
    g = svg.Geom(B=1, H=c["H"], d=c["d"], N=c["N"], F=c["F"], T=c["T"], a1=c["a1"], a2=c["a2"], window=c["F"],
                 stripe=512)
    q, k, v = (to_device(inp[n][None], torch.bfloat16) for n in "qkv")
    rows = torch.from_numpy(inp["rows"]).cuda()
    flags = svg.FP8_SCORES | svg.FP8_PV
    ws = svg.alloc_workspace(g, svg.BF16, rows.numel(), flags)
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    labels = torch.full((g.H,), -1, dtype=torch.int32, device="cuda")
    stats = torch.zeros(g.H * 3, dtype=torch.float32, device="cuda")
    print("\n[fp8 P.V layer hunyuanvideo shape]", flush=True)
    svg.svg_layer_forward(g, q, k, v, o, ws, rows=rows, labels_out=labels, stats_out=stats, flags=flags)
    torch.cuda.synchronize()
    lab = labels.cpu().numpy()
    assert np.array_equal(lab, inp["kinds"])
    og = ogeom(g)
    rng = np.random.default_rng(19)
    check_rows = np.unique(np.concatenate([[0, g.L - 1], rng.choice(g.L, 24, replace=False)]))
    got = o[0].float().cpu().numpy()
    for h in (0, 1):
        _, _, _, _, qd, kd = oracle_quant(g, int(lab[h]), inp["q"][h], inp["k"][h])
        cv, s = fp8.quantize_head(inp["v"][h])
        vd = (fp8.e4m3_decode(cv) * s).astype(np.float32)
        worst = check_fp8_pv_rows(got[h][check_rows], qd, kd, vd, og, int(lab[h]), scale_of(g), check_rows,
                                  f"fp8 P.V layer head {h}")
        print(f"  head {h} (label {lab[h]}): worst err / bound {worst:.3f}", flush=True)


def test_fp8_strided_equals_contiguous():
    """Token-interleaved [B, L, H, d] inputs (B = 2): Q8, K8, V8 codes, scales
    and both FP8 attention outputs bit-identical to the contiguous run."""
    B, H, N, F, T, d = 2, 3, 4, 70, 6, 128
    modes = [svg.SPATIAL, svg.TEMPORAL, svg.FULL, svg.WINDOW, svg.STRIPE, svg.TEMPORAL]
    g = svg.Geom(B=B, H=H, d=d, N=N, F=F, T=T, a1=2, a2=8, window=50, stripe=64)
    L = g.L
    inp = S.small_config(N, F, T, B * H, d, 2, 8, [PLANT[m] for m in modes], seed=31, window=50, stripe=64)
    modes_t = torch.tensor(modes, dtype=torch.int32, device="cuda")
    BM, BN = svg.svg_tile_config(svg.BF16, d)
    nq = -(-L // BM)
    ranges = torch.empty(B * H * nq * 4, dtype=torch.int32, device="cuda")
    order = torch.empty(B * H, dtype=torch.int32, device="cuda")
    svg.svg_build_blocks(g, modes_t, BM, BN, ranges, order)
    print("\n[fp8 strided vs contiguous]", flush=True)
    res = []
    for interleave in (False, True):
        if interleave:
            q, k, v = (torch.from_numpy(np.ascontiguousarray(inp[n].reshape(B, H, L, d).transpose(0, 2, 1, 3)))
                       .to(torch.bfloat16).cuda().permute(0, 2, 1, 3) for n in "qkv")
            mk_o = lambda: torch.full((B, L, H, d), float("nan"), dtype=torch.bfloat16,
                                      device="cuda").permute(0, 2, 1, 3)
        else:
            q, k, v = (to_device(inp[n].reshape(B, H, L, d), torch.bfloat16) for n in "qkv")
            mk_o = lambda: torch.full((B, H, L, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        q8, sq, k8, sk = quantize_on_gpu(g, q, k, modes_t)
        v8, sv = quantize_v_on_gpu(g, v, modes_t)
        o1, o2 = mk_o(), mk_o()
        svg.svg_sparse_attention_fp8(g, q8, sq, k8, sk, v, o1, modes_t, ranges, order)
        svg.svg_sparse_attention_fp8_pv(g, q8, sq, k8, sk, v8, sv, o2, modes_t, ranges, order)
        torch.cuda.synchronize()
        res.append([t.float().cpu().numpy() for t in (q8, sq, k8, sk, v8, sv, o1, o2)])
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
