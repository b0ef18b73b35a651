"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/svg.h declares, and rejects invalid arguments with the
documented status before it makes any HIP call (so nothing is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_video_svg_amd as svg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svg.h")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = range(5)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svg2?_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["svg_abi_version", "svg_last_error", "svg_tile_config", "svg_workspace_bytes", "svg_profile_heads",
              "svg_build_blocks", "svg_layout_permute", "svg_sparse_attention", "svg_layer_forward"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(svg.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", svg.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (svg2?_\w+)", out))
    assert set(declared_functions()) <= exported
    assert svg.svg_abi_version() == 1


def test_python_binding_has_the_same_names():
    for n in declared_functions():
        assert callable(getattr(svg, n)), n


def test_tile_config():
    bm, bn = svg.svg_tile_config(svg.BF16, 128)
    assert bn == 64 and bm % 32 == 0 and bm >= 128
    assert svg.svg_tile_config(svg.BF16, 64) == (bm, bn)
    assert svg.svg_tile_config(svg.F32, 64) == (64, 64)
    with pytest.raises(svg.SvgError) as e:
        svg.svg_tile_config(svg.BF16, 96)
    assert e.value.status == E_UNSUPPORTED
    with pytest.raises(svg.SvgError) as e:
        svg.svg_tile_config(7, 64)
    assert e.value.status == E_INVALID


def geom(**kw):
    g = dict(B=1, H=2, d=128, N=4, F=64, T=0, a1=2, a2=8, window=64, stripe=16, scale=0.0)
    g.update(kw)
    return svg.Geom(**g)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), E_INVALID), (dict(H=0), E_INVALID), (dict(d=96), E_UNSUPPORTED), (dict(N=0), E_INVALID),
    (dict(F=0), E_INVALID), (dict(T=-1), E_INVALID), (dict(a1=0), E_INVALID), (dict(a2=0), E_INVALID),
    (dict(window=0), E_INVALID), (dict(stripe=0), E_INVALID), (dict(scale=-1.0), E_INVALID),
    (dict(scale=float("inf")), E_INVALID), (dict(H=5000), E_UNSUPPORTED), (dict(N=1 << 16, F=1 << 15), E_UNSUPPORTED),
])
def test_geometry_validation(kw, status):
    with pytest.raises(svg.SvgError) as e:
        svg.svg_workspace_bytes(geom(**kw), svg.BF16, 0, 0)
    assert e.value.status == status
    assert svg.svg_last_error()


def test_workspace_bytes_grows_with_rows_and_explicit_permutation():
    g = geom()
    a = svg.svg_workspace_bytes(g, svg.BF16, 0, svg.VIRTUAL_PERMUTE)
    b = svg.svg_workspace_bytes(g, svg.BF16, 16, svg.VIRTUAL_PERMUTE)
    c = svg.svg_workspace_bytes(g, svg.BF16, 16, 0)
    assert 0 < a < b < c
    L = g.L
    # the explicit layout holds token-major copies of K and V (bf16)
    assert c - b >= 2 * g.H * L * g.d * 2
    with pytest.raises(svg.SvgError):
        svg.svg_workspace_bytes(g, svg.BF16, g.N * g.F + 1, 0)
    with pytest.raises(svg.SvgError):
        svg.svg_workspace_bytes(g, svg.BF16, 0, 8)


# Raw calls with fake (aligned, never dereferenced) device addresses: each
# must fail in validation, before any HIP call.
A = 0x10000  # 16-byte aligned fake address


def raw():
    return svg._lib()


def strides(b=4 * 64 * 128, h=64 * 128 * 0 + 256 * 128, x=128):
    return svg._Strides(b, h, x)


BM_BF16, BN_BF16 = svg.svg_tile_config(svg.BF16, 128)


# distinct fake addresses of the tensors of one call
Q, K, V, O, QP, KP, VP, OP = (A + i * 0x1000000 for i in range(8))


def call_attention(g, din=svg.BF16, dout=svg.BF16, q=Q, s=None, o=O, so=None, modes=A, ranges=A, order=A,
                   BM=BM_BF16, BN=BN_BF16, flags=0, qp=QP, kp=KP, sp=None, op=OP):
    gc = g.c()
    s = s or strides()
    so = so or strides()
    sp = sp or strides()
    return raw().svg_sparse_attention(ctypes.byref(gc), din, dout, q, K, V, s, qp, kp, VP, sp, o, so, op, sp, modes,
                                      ranges, order, BM, BN, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_INVALID), (dict(q=A + 8), E_INVALID), (dict(o=None), E_INVALID),
    (dict(modes=None), E_INVALID), (dict(ranges=None), E_INVALID), (dict(order=None), E_INVALID),
    (dict(BM=64), E_UNSUPPORTED), (dict(BN=128), E_UNSUPPORTED), (dict(din=svg.F32, dout=svg.BF16), E_UNSUPPORTED),
    (dict(din=5), E_INVALID), (dict(flags=4), E_INVALID), (dict(kp=None), E_INVALID), (dict(qp=A + 8), E_INVALID),
    (dict(s=svg._Strides(0, 0, 64)), E_INVALID), (dict(s=svg._Strides(0, 0, 132)), E_INVALID),
    (dict(so=svg._Strides(-8, 0, 128)), E_INVALID),
])
def test_attention_validation(kw, status):
    assert call_attention(geom(), **kw) == status
    assert svg.svg_last_error()


def test_outputs_must_not_overlap_inputs():
    """An output starting at an input's address is rejected before any HIP
    call.  Each call also carries an argument error that validation reports
    after the overlap check, so none of them could reach the device even if
    the overlap went unnoticed."""
    g = geom().c()
    L = raw()
    s = strides()

    def rejected_for_overlap(status):
        return status == E_INVALID and "overlap" in svg.svg_last_error()

    # attention (modes NULL: checked after the overlap)
    for kw in (dict(o=Q), dict(o=KP), dict(op=V), dict(op=O)):
        assert rejected_for_overlap(call_attention(geom(), modes=None, **kw)), kw
    assert call_attention(geom(), modes=None) == E_INVALID and "modes" in svg.svg_last_error()
    # the layer (rows NULL: checked after the overlap)
    n_need = svg.svg_workspace_bytes(geom(), svg.BF16, 8, 0)
    for o in (Q, K, V):
        assert rejected_for_overlap(L.svg_layer_forward(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, o, s, None, 8,
                                                        0.05, None, A, A, 0, A, n_need, None))
        assert rejected_for_overlap(L.svg_layer_forward_noalloc(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, o, s,
                                                                None, 8, 0.05, None, A, A, 0, None))
    # fp8 quantisation and attention, SVG2 forward
    # (sk / sv NULL: checked after the overlap)
    assert rejected_for_overlap(L.svg_quantize_qk(ctypes.byref(g), svg.BF16, Q, K, s, A, Q, A, KP, None, None))
    assert rejected_for_overlap(L.svg_quantize_qk(ctypes.byref(g), svg.BF16, Q, K, s, A, QP, A, QP, None, None))
    assert rejected_for_overlap(L.svg_quantize_v(ctypes.byref(g), svg.BF16, V, s, A, V, None, None))
    # (modes / mu_q NULL: checked after the overlap)
    assert rejected_for_overlap(L.svg_sparse_attention_fp8(ctypes.byref(g), svg.BF16, QP, A, KP, A, V, s, V, s, None,
                                                           A, A, BM_BF16, BN_BF16, None))
    assert rejected_for_overlap(L.svg_sparse_attention_fp8_pv(ctypes.byref(g), svg.BF16, QP, A, KP, A, VP, A, KP, s,
                                                              None, A, A, BM_BF16, BN_BF16, None))
    prm = svg._Svg2Params(32, 32, 2, 0.9)
    assert rejected_for_overlap(L.svg2_forward(ctypes.byref(g), ctypes.byref(prm), svg.BF16, svg.BF16, Q, K, V, s, K,
                                               s, 0, None, A, None, A, 1 << 40, None))


def test_profile_validation():
    g = geom().c()
    L = raw()
    s = strides()
    base = dict(q=A, rows=A, n=8, fb=0.05, labels=A, stats=A, ws=A, wsb=1 << 30)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return L.svg_profile_heads(ctypes.byref(g), svg.BF16, a["q"], A, A, s, a["rows"], a["n"], a["fb"],
                                   a["labels"], a["stats"], a["ws"], a["wsb"], None)

    assert call(rows=None) == E_INVALID
    assert call(n=0) == E_INVALID
    assert call(n=4 * 64 + 1) == E_INVALID
    assert call(fb=0.0) == E_INVALID
    assert call(fb=float("nan")) == E_INVALID
    assert call(labels=None) == E_INVALID
    assert call(ws=None) == E_INVALID
    assert call(ws=A + 16) == E_INVALID
    assert call(wsb=16) == E_WORKSPACE


def test_blocks_permute_layer_validation():
    g = geom().c()
    L = raw()
    assert L.svg_build_blocks(ctypes.byref(g), A, 100, 64, A, A, None) == E_UNSUPPORTED
    assert L.svg_build_blocks(ctypes.byref(g), None, 128, 64, A, A, None) == E_INVALID
    assert L.svg_build_blocks(None, A, 128, 64, A, A, None) == E_INVALID
    s = strides()
    assert L.svg_layout_permute(ctypes.byref(g), svg.BF16, A, s, A, s, None, 0, None) == E_INVALID  # overlap
    assert L.svg_layout_permute(ctypes.byref(g), svg.BF16, None, s, A, s, None, 0, None) == E_INVALID
    assert L.svg_layout_permute(ctypes.byref(g), 3, A, s, A + 4096, s, None, 0, None) == E_INVALID
    # layer: too small a workspace, bad flags, missing labels when profiling
    assert L.svg_layer_forward(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, O, s, A, 8, 0.05, None, A, A, 0, A,
                               1024, None) == E_WORKSPACE
    assert L.svg_layer_forward(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, O, s, A, 8, 0.05, None, A, A, 2, A,
                               1 << 40, None) == E_INVALID
    assert L.svg_layer_forward(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, O, s, A, 8, 0.05, None, None, A, 0,
                               A, 1 << 40, None) == E_INVALID


def test_search_validation():
    g = geom().c()
    L = raw()
    s = strides()
    base = dict(dt=svg.BF16, rows=A, n=8, lam=0.5, eps=1.0, pen=0, modes=A, stats=A, ws=A, wsb=1 << 30)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return L.svg_search_modes(ctypes.byref(g), a["dt"], A, A, A, s, a["rows"], a["n"], a["lam"], a["eps"],
                                  a["pen"], a["modes"], a["stats"], a["ws"], a["wsb"], None)

    assert call(dt=svg.F32) == E_UNSUPPORTED
    assert call(rows=None) == E_INVALID
    assert call(n=0) == E_INVALID
    assert call(lam=-0.1) == E_INVALID
    assert call(lam=float("inf")) == E_INVALID
    assert call(eps=float("nan")) == E_INVALID
    assert call(pen=2) == E_INVALID
    assert call(modes=None) == E_INVALID
    assert call(stats=None) == E_INVALID
    assert call(ws=A + 16) == E_INVALID
    assert call(wsb=16) == E_WORKSPACE
    gg = geom()
    plain = svg.svg_workspace_bytes(gg, svg.BF16, 16, svg.VIRTUAL_PERMUTE)
    search = svg.svg_workspace_bytes(gg, svg.BF16, 16, svg.MODE_SEARCH | svg.VIRTUAL_PERMUTE)
    assert search > plain
    with pytest.raises(svg.SvgError) as e:
        svg.svg_workspace_bytes(gg, svg.F32, 16, svg.MODE_SEARCH)
    assert e.value.status == E_UNSUPPORTED


def test_svg2_validation():
    g = geom().c()
    L = raw()
    s = strides()
    gg = geom()
    need = svg.svg2_workspace_bytes(gg, svg.Svg2Params(32, 48, 2, 0.9))
    assert need > svg.svg2_workspace_bytes(gg, svg.Svg2Params(32, 32, 2, 0.9))
    base = dict(Cq=32, Ck=48, it=2, p=0.9, din=svg.BF16, dout=svg.BF16, flags=0, mq=A, mk=A, ws=A, wsb=need)

    def fwd(**kw):
        a = dict(base)
        a.update(kw)
        prm = svg._Svg2Params(a["Cq"], a["Ck"], a["it"], a["p"])
        return L.svg2_forward(ctypes.byref(g), ctypes.byref(prm), a["din"], a["dout"], Q, K, V, s, O, s, a["flags"],
                              a["mq"], a["mk"], None, a["ws"], a["wsb"], None)

    assert fwd(Cq=0) == E_INVALID
    assert fwd(Ck=1025) == E_UNSUPPORTED
    assert fwd(Cq=gg.L + 1) in (E_INVALID, E_UNSUPPORTED)
    assert fwd(it=0) == E_INVALID
    assert fwd(p=0.0) == E_INVALID
    assert fwd(p=float("nan")) == E_INVALID
    assert fwd(din=svg.F32) == E_UNSUPPORTED
    assert fwd(dout=9) == E_INVALID
    assert fwd(flags=2) == E_INVALID
    assert fwd(mq=None) == E_INVALID
    assert fwd(mk=None) == E_INVALID
    assert fwd(ws=A + 16) == E_INVALID
    assert fwd(wsb=need - 1) == E_WORKSPACE

    def km(C=32, it=2, flags=0, wsb=need, dt=svg.BF16, mu=A, lab=A, perm=A, start=A):
        return L.svg2_kmeans(ctypes.byref(g), dt, A, s, C, it, flags, mu, lab, perm, start, A, wsb, None)

    assert km(C=0) == E_INVALID
    assert km(it=0) == E_INVALID
    assert km(flags=4) == E_INVALID
    assert km(dt=svg.F32) == E_UNSUPPORTED
    assert km(mu=None) == E_INVALID and km(lab=None) == E_INVALID
    assert km(perm=None) == E_INVALID and km(start=None) == E_INVALID
    assert km(wsb=16) == E_WORKSPACE


def test_fp8_pv_validation():
    g = geom().c()
    L = raw()
    s = strides()
    assert L.svg_quantize_v(ctypes.byref(g), svg.F32, V, s, A, VP, A, None) == E_UNSUPPORTED
    assert L.svg_quantize_v(ctypes.byref(g), svg.BF16, V, s, A, None, A, None) == E_INVALID
    assert L.svg_quantize_v(ctypes.byref(g), svg.BF16, V, s, A, VP, None, None) == E_INVALID
    assert L.svg_quantize_v(ctypes.byref(g), svg.BF16, V, s, None, VP, A, None) == E_INVALID

    def att(BM=BM_BF16, BN=BN_BF16, v8=VP, sv=A, out=svg.BF16):
        return L.svg_sparse_attention_fp8_pv(ctypes.byref(g), out, QP, A, KP, A, v8, sv, O, s, A, A, A, BM, BN, None)

    assert att(BM=BM_BF16 // 2) == E_UNSUPPORTED
    assert att(v8=None) == E_INVALID
    assert att(sv=None) == E_INVALID
    assert att(out=9) == E_INVALID
    gg = geom()
    with pytest.raises(svg.SvgError) as e:
        svg.svg_workspace_bytes(gg, svg.BF16, 16, svg.FP8_PV)
    assert e.value.status == E_INVALID
    a = svg.svg_workspace_bytes(gg, svg.BF16, 16, svg.FP8_SCORES)
    b = svg.svg_workspace_bytes(gg, svg.BF16, 16, svg.FP8_SCORES | svg.FP8_PV)
    nkt = -(-gg.L // 64)
    assert b - a >= gg.H * nkt * gg.d * 64


def test_noalloc_layer_validation():
    """svg_layer_forward_noalloc rejects on the host, before any HIP call: fp8
    flags, a layer whose workspace exceeds the fixed scratch even with one key
    slice, and the same argument errors as svg_layer_forward."""
    L = raw()
    s = strides()
    g = geom().c()
    assert svg.svg_noalloc_scratch_bytes() == 64 << 20
    assert L.svg_layer_forward_noalloc(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, O, s, A, 8, 0.05, None, A, A,
                                       svg.FP8_SCORES, None) == E_UNSUPPORTED
    assert L.svg_layer_forward_noalloc(ctypes.byref(g), svg.BF16, svg.BF16, Q, K, V, s, O, s, A, 8, 0.05, None, None,
                                       A, 0, None) == E_INVALID
    assert L.svg_layer_forward_noalloc(ctypes.byref(g), svg.BF16, svg.BF16, None, K, V, s, O, s, A, 8, 0.05, None, A,
                                       A, 0, None) == E_INVALID
    # 64 heads x 2048 tokens, all rows profiled: partials 64*2048*3*66*4 bytes > 64 MiB at one slice
    big = svg.Geom(B=1, H=64, d=64, N=2, F=1024, T=0, a1=1, a2=4, window=64, stripe=64).c()
    sb = svg._Strides(64 * 2048 * 64, 2048 * 64, 64)
    assert L.svg_layer_forward_noalloc(ctypes.byref(big), svg.BF16, svg.BF16, Q, K, V, sb, O, sb, A, 2048, 0.05, None,
                                       A, A, 0, None) == E_WORKSPACE
    assert "scratch" in svg.svg_last_error()
