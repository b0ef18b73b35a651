"""Two layers in flight at once on two streams (default priority), each with
its own inputs, outputs and workspace: every call gives the same bits as the
same call run alone (marked gpu).  The library keeps no per-call state
outside the caller's buffers (the device topology and kernel attributes it
caches are written once), so calls on different streams do not interact.
"""
import numpy as np
import pytest

import sparse_attention_video_svg_amd as svg
import svg_synth as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KINDS = [S.SPATIAL, S.TEMPORAL, S.UNSTRUCTURED, S.TEMPORAL, S.SPATIAL, S.TEMPORAL]


def _case(g, seed, count, flags):
    inp = S.small_config(g.N, g.F, g.T, g.H, g.d, g.a1, g.a2, KINDS, seed=seed)
    q, k, v = (torch.from_numpy(inp[n][None]).cuda().to(torch.bfloat16) for n in "qkv")
    rows = torch.from_numpy(svg.svg_sample_rows(g, count, seed)).cuda()
    ws = svg.alloc_workspace(g, svg.BF16, count, flags)
    return dict(q=q, k=k, v=v, rows=rows, ws=ws, flags=flags)


def _run(g, c, stream=None):
    o = torch.full(c["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lab = torch.full((g.H,), -1, dtype=torch.int32, device="cuda")
    st = torch.full((g.H * 3,), float("nan"), dtype=torch.float32, device="cuda")
    svg.svg_layer_forward(g, c["q"], c["k"], c["v"], o, c["ws"], rows=c["rows"], labels_out=lab, stats_out=st,
                          flags=c["flags"], stream=stream)
    return o, lab, st


def _host(r):
    o, lab, st = r
    return o.view(torch.int16).cpu().numpy(), lab.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128])
def test_two_streams_equal_alone(d):
    g = svg.Geom(B=1, H=len(KINDS), d=d, N=8, F=600, T=32, a1=2, a2=50)
    print(f"\n[two streams: d {d}]", flush=True)
    cases = [_case(g, 300 + d, 48, 0), _case(g, 400 + d, 48, svg.VIRTUAL_PERMUTE)]
    alone = []
    for c in cases:
        r = _run(g, c)
        torch.cuda.synchronize()
        alone.append(_host(r))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        outs = []
        # interleave the launches of the two layers on their streams
        for c, s in zip(cases, streams):
            with torch.cuda.stream(s):
                outs.append(_run(g, c, stream=s))
        torch.cuda.synchronize()
        for i, r in enumerate(outs):
            got, want = _host(r), alone[i]
            assert np.array_equal(got[1], want[1]), (rep, i)
            np.testing.assert_array_equal(got[2], want[2])
            assert np.array_equal(got[0], want[0]), f"repeat {rep}, layer {i}: outputs differ from the call alone"
