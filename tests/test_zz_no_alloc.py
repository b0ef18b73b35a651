"""svg_layer_forward_noalloc (workspace in the library's fixed per-device
scratch, no allocation in the call) against svg_layer_forward with a caller
workspace, on two calls in a row, the second with a smaller input (marked
gpu).

Labels and outputs must be bit-identical (the same kernels run on the same
inputs; the fixed-scratch call always takes the index-map layout, which the
workload tests hold bit-identical to the explicit one).  The profiling
statistics may come from fewer key slices when the scratch cannot hold the
default number of partials (the HunyuanVideo-shaped layer drops to one
slice), so they are held at the statistics bar (2 % relative, 1e-4 absolute).
"""
import ctypes

import numpy as np
import pytest

import sparse_attention_video_svg_amd as svg
import svg_synth as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _geom_of(c):
    return svg.Geom(B=1, H=c["H"], d=c["d"], N=c["N"], F=c["F"], T=c["T"], a1=c["a1"], a2=c["a2"],
                    window=c.get("window", c["F"]), stripe=c.get("stripe", 512))


def _both(g, inp, rows_np):
    dev = "cuda"
    q, k, v = (torch.from_numpy(inp[n]).to(dev).to(torch.bfloat16)[None] for n in "qkv")
    rows = torch.from_numpy(rows_np.astype(np.int32)).to(dev)
    res = []
    for noalloc in (False, True):
        o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=dev)
        labels = torch.full((g.H,), -1, dtype=torch.int32, device=dev)
        stats = torch.full((g.H * 3,), float("nan"), dtype=torch.float32, device=dev)
        if noalloc:
            svg.svg_layer_forward_noalloc(g, q, k, v, o, rows=rows, labels_out=labels, stats_out=stats)
        else:
            ws = svg.alloc_workspace(g, svg.BF16, rows.numel(), svg.VIRTUAL_PERMUTE)
            svg.svg_layer_forward(g, q, k, v, o, ws, rows=rows, labels_out=labels, stats_out=stats,
                                  flags=svg.VIRTUAL_PERMUTE)
        torch.cuda.synchronize()
        res.append((o.view(torch.int16).cpu().numpy(), labels.cpu().numpy(), stats.cpu().numpy()))
    return res


def test_noalloc_equals_layer_forward_two_calls():
    # call 1: the HunyuanVideo-shaped layer (its default profiling partials
    # exceed the scratch, so the slice count is capped)
    c = S.WORKLOADS[S.HUNYUANVIDEO]
    print(f"\n[noalloc call 1: {c['name']}]", flush=True)
    inp = S.make_inputs(S.HUNYUANVIDEO)
    g = _geom_of(c)
    (o_ref, lab_ref, st_ref), (o, lab, st) = _both(g, inp, inp["rows"])
    assert np.array_equal(lab, lab_ref), (lab, lab_ref)
    assert np.array_equal(o, o_ref), "outputs differ"
    np.testing.assert_allclose(st, st_ref, rtol=2e-2, atol=1e-4)
    del inp
    # call 2: a smaller layer with a text prefix, d 64; the scratch still holds
    # the first call's contents
    N, F, T, H, d, a1, a2 = 5, 320, 24, 4, 64, 2, 20
    print(f"[noalloc call 2: {N}x{F} + {T} text, {H} heads, d {d}]", flush=True)
    kinds = [S.SPATIAL, S.TEMPORAL, S.TEMPORAL, S.SPATIAL]
    inp = S.small_config(N, F, T, H, d, a1, a2, kinds, seed=77)
    g = svg.Geom(B=1, H=H, d=d, N=N, F=F, T=T, a1=a1, a2=a2, window=F, stripe=64)
    rows_np = S.sample_rows(N, F, T, 0.05, 78)
    (o_ref, lab_ref, st_ref), (o, lab, st) = _both(g, inp, rows_np)
    assert np.array_equal(lab, lab_ref), (lab, lab_ref)
    assert np.array_equal(lab, np.array(kinds, dtype=np.int32))
    assert np.array_equal(o, o_ref), "outputs differ"
    np.testing.assert_allclose(st, st_ref, rtol=2e-2, atol=1e-4)


def test_noalloc_rejects_before_enqueueing():
    """Host-side rejections: fp8 flags, and a layer whose workspace cannot fit
    the scratch even with one key slice."""
    g = svg.Geom(B=1, H=4, d=64, N=4, F=64, T=0, a1=1, a2=4, window=64, stripe=64)
    x = torch.zeros((1, g.H, g.L, g.d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    rows = torch.arange(0, g.L, dtype=torch.int32, device="cuda")
    lab = torch.empty(g.H, dtype=torch.int32, device="cuda")
    st = torch.empty(g.H * 3, dtype=torch.float32, device="cuda")
    with pytest.raises(svg.SvgError) as e:
        svg.svg_layer_forward_noalloc(g, x, x, x, o, rows=rows, labels_out=lab, stats_out=st, flags=svg.FP8_SCORES)
    assert e.value.status == 2
    # 64 heads, 2048 tokens, every row sampled: the profiling partials alone
    # (one key slice) are 64*2048*3*66*4 bytes = 104 MB > 64 MiB
    big = svg.Geom(B=1, H=64, d=64, N=2, F=1024, T=0, a1=1, a2=4, window=64, stripe=64)
    assert svg.svg_noalloc_scratch_bytes() < big.H * big.L * 3 * 66 * 4
    xb = torch.zeros((1, big.H, big.L, 64), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty_like(xb)
    rows_b = torch.arange(0, big.L, dtype=torch.int32, device="cuda")
    lab_b = torch.empty(big.H, dtype=torch.int32, device="cuda")
    st_b = torch.empty(big.H * 3, dtype=torch.float32, device="cuda")
    with pytest.raises(svg.SvgError) as e:
        svg.svg_layer_forward_noalloc(big, xb, xb, xb, ob, rows=rows_b, labels_out=lab_b, stats_out=st_b)
    assert e.value.status == 3
