"""Sparse VideoGen spatial/temporal sparse attention on MI355X (gfx950).

Thin Python binding of ``libsvg.so`` (C ABI in ``include/svg.h``): argument
marshalling only.  Every step of the path (profiling, tile lists, layout
transformation, sparse attention) runs in the library's HIP kernels; PyTorch
only provides device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.

Function names equal the C entry points.  Tensors are ``[B, H, L, d]`` with
``d`` contiguous, ``L = T + N*F``; dtype bfloat16 or float32.
"""
import ctypes
import dataclasses
import math
import os

__all__ = [
    "SPATIAL", "TEMPORAL", "FULL", "SKIP", "WINDOW", "STRIPE", "F32", "BF16", "VIRTUAL_PERMUTE", "MODE_SEARCH",
    "FP8_SCORES", "SEARCH_CANDIDATES", "Geom", "SvgError", "svg_abi_version", "svg_last_error", "svg_tile_config",
    "svg_sample_rows",
    "svg_workspace_bytes", "svg_profile_heads", "svg_search_modes", "svg_build_blocks", "svg_layout_permute",
    "svg_sparse_attention", "svg_quantize_qk", "svg_sparse_attention_fp8", "svg_quantize_v",
    "svg_sparse_attention_fp8_pv", "FP8_PV", "svg_layer_forward", "svg_layer_forward_noalloc",
    "svg_noalloc_scratch_bytes", "library_path",
    "Svg2Params", "SVG2_INIT_GIVEN", "svg2_workspace_bytes", "svg2_kmeans", "svg2_forward",
]

SPATIAL, TEMPORAL, FULL, SKIP, WINDOW, STRIPE = range(6)
F32, BF16 = 0, 1
VIRTUAL_PERMUTE = 1
MODE_SEARCH = 2  # svg_workspace_bytes: size for svg_search_modes
FP8_SCORES = 4   # svg_layer_forward: scores on FP8 E4M3 Q and K
FP8_PV = 8       # with FP8_SCORES: P.V on FP8 E4M3 weights and V as well
SEARCH_CANDIDATES = (SKIP, WINDOW, TEMPORAL, STRIPE)  # order of svg_search_modes' stats

# The library trusts device-side contents (sampled rows, modes, tile ranges,
# head order).  With DEBUG true (or SVG_DEBUG=1 in the environment) the
# binding copies them to the host and validates them before each call; this
# synchronises the device.
DEBUG = os.environ.get("SVG_DEBUG", "") not in ("", "0")

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVG_LIBRARY may point at another build of the same library (A/B timing).
_LIB_PATH = os.environ.get("SVG_LIBRARY") or os.path.join(_HERE, "libsvg.so")


def library_path():
    return _LIB_PATH


class SvgError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"svg status {status}: {msg}")
        self.status = status


class _Geom(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("F", ctypes.c_int32), ("T", ctypes.c_int32), ("a1", ctypes.c_int32), ("a2", ctypes.c_int32),
                ("window", ctypes.c_int32), ("stripe", ctypes.c_int32), ("scale", ctypes.c_float)]


class _Svg2Params(ctypes.Structure):
    _fields_ = [("C_q", ctypes.c_int32), ("C_k", ctypes.c_int32), ("iters", ctypes.c_int32), ("p", ctypes.c_float)]


@dataclasses.dataclass
class Svg2Params:
    """SVG2 clustering and selection: clusters of Q and K per head, Lloyd
    iterations, top-p threshold."""
    C_q: int = 256
    C_k: int = 256
    iters: int = 3
    p: float = 0.9

    def c(self):
        return _Svg2Params(self.C_q, self.C_k, self.iters, float(self.p))


SVG2_INIT_GIVEN = 1


class _Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("x", ctypes.c_int64)]


@dataclasses.dataclass
class Geom:
    """Geometry of one attention layer: B x H heads of width d over T text
    tokens followed by N frames of F tokens.  a1 / a2: spatial / temporal
    thresholds; window / stripe: Sparse-vDiT diagonal width and stripe keys;
    scale 0 means 1/sqrt(d)."""
    B: int
    H: int
    d: int
    N: int
    F: int
    T: int = 0
    a1: int = 1
    a2: int = 1
    window: int = 1
    stripe: int = 1
    scale: float = 0.0

    @property
    def L(self):
        return self.T + self.N * self.F

    def c(self):
        return _Geom(self.B, self.H, self.d, self.N, self.F, self.T, self.a1, self.a2, self.window,
                     self.stripe, float(self.scale))


_lib_handle = None


def _check_single_hip_runtime():
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError("two HIP runtimes are loaded in this process (" + ", ".join(sorted(real)) +
                           "); import torch before anything that loads libamdhip64")


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python -m sparse_attention_video_svg_amd._build")
        # torch brings its own HIP runtime (same soname as the system one the
        # library is linked against).  Load it first so that the library binds
        # to that one copy: two runtimes in one process do not share devices,
        # streams or allocations.
        import torch  # noqa: F401
        L = ctypes.CDLL(_LIB_PATH)
        _check_single_hip_runtime()
        P = ctypes.POINTER
        g = P(_Geom)
        S = _Strides
        vp = ctypes.c_void_p
        i32 = ctypes.c_int32
        sig = {
            "svg_abi_version": ([], i32),
            "svg_last_error": ([], ctypes.c_char_p),
            "svg_tile_config": ([i32, i32, P(i32), P(i32)], i32),
            "svg_sample_rows": ([g, i32, ctypes.c_uint64, P(i32)], i32),
            "svg_workspace_bytes": ([g, i32, i32, i32, P(ctypes.c_size_t)], i32),
            "svg_profile_heads": ([g, i32, vp, vp, vp, S, vp, i32, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp],
                                  i32),
            "svg_search_modes": ([g, i32, vp, vp, vp, S, vp, i32, ctypes.c_float, ctypes.c_float, i32, vp, vp, vp,
                                  ctypes.c_size_t, vp], i32),
            "svg_build_blocks": ([g, vp, i32, i32, vp, vp, vp], i32),
            "svg_layout_permute": ([g, i32, vp, S, vp, S, vp, i32, vp], i32),
            "svg_sparse_attention": ([g, i32, i32, vp, vp, vp, S, vp, vp, vp, S, vp, S, vp, S, vp, vp, vp, i32, i32,
                                      i32, vp], i32),
            "svg_quantize_qk": ([g, i32, vp, vp, S, vp, vp, vp, vp, vp, vp], i32),
            "svg_sparse_attention_fp8": ([g, i32, vp, vp, vp, vp, vp, S, vp, S, vp, vp, vp, i32, i32, vp], i32),
            "svg_quantize_v": ([g, i32, vp, S, vp, vp, vp, vp], i32),
            "svg_sparse_attention_fp8_pv": ([g, i32, vp, vp, vp, vp, vp, vp, vp, S, vp, vp, vp, i32, i32, vp], i32),
            "svg2_workspace_bytes": ([g, P(_Svg2Params), P(ctypes.c_size_t)], i32),
            "svg2_kmeans": ([g, i32, vp, S, i32, i32, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp], i32),
            "svg2_forward": ([g, P(_Svg2Params), i32, i32, vp, vp, vp, S, vp, S, i32, vp, vp, vp, vp,
                              ctypes.c_size_t, vp], i32),
            "svg_layer_forward": ([g, i32, i32, vp, vp, vp, S, vp, S, vp, i32, ctypes.c_float, vp, vp, vp, i32, vp,
                                   ctypes.c_size_t, vp], i32),
            "svg_layer_forward_noalloc": ([g, i32, i32, vp, vp, vp, S, vp, S, vp, i32, ctypes.c_float, vp, vp, vp,
                                           i32, vp], i32),
            "svg_noalloc_scratch_bytes": ([], ctypes.c_size_t),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib_handle = L
    return _lib_handle


def _check(status):
    if status != 0:
        raise SvgError(status, svg_last_error())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t):
    """Element strides (b, h, x) of a [B, H, L, d] tensor with d contiguous."""
    if t is None:
        return _Strides(0, 0, 0)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("tensors must be [B, H, L, d] with d contiguous")
    return _Strides(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_shape(geom, t, name):
    if tuple(t.shape) != (geom.B, geom.H, geom.L, geom.d):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(geom.B, geom.H, geom.L, geom.d)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _check_vec(t, name, dtype, n, optional=False):
    """Metadata of a small device vector: dtype, contiguity, length >= n."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, needs {n}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _t_i32():
    import torch
    return torch.int32


def _t_f32():
    import torch
    return torch.float32


def _check_tile_args(geom, BM, BN, modes, ranges, head_order):
    BH = geom.B * geom.H
    _check_vec(modes, "modes", _t_i32(), BH)
    _check_vec(ranges, "ranges", _t_i32(), BH * -(-geom.L // BM) * 4)
    _check_vec(head_order, "head_order", _t_i32(), BH)
    if DEBUG:
        _debug_modes(geom, modes)
        _debug_tiles(geom, BM, BN, ranges, head_order)


def _debug_rows(geom, rows):
    """Sampled rows: strictly ascending video rows in [T, L)."""
    r = rows.detach().to("cpu").long()
    if r.numel() == 0:
        raise ValueError("rows is empty")
    if int(r[0]) < geom.T or int(r[-1]) >= geom.L:
        raise ValueError(f"rows must lie in [T, L) = [{geom.T}, {geom.L}), got [{int(r[0])}, {int(r[-1])}]")
    if r.numel() > 1 and not bool((r[1:] > r[:-1]).all()):
        raise ValueError("rows must be strictly ascending (distinct, sorted)")


def _debug_modes(geom, modes):
    m = modes.detach().to("cpu")[: geom.B * geom.H]
    bad = (m < SPATIAL) | (m > STRIPE)
    if bool(bad.any()):
        i = int(bad.nonzero()[0])
        raise ValueError(f"modes[{i}] = {int(m[i])} is not a mode (0..5)")


def _debug_tiles(geom, BM, BN, ranges, head_order):
    """Tile ranges: per (head, query tile) [x, y) U [z, w) within the key
    tiles, the second empty (z = w) or after the first (y <= z); head order:
    a permutation of the heads."""
    import torch
    BH = geom.B * geom.H
    nq, nk = -(-geom.L // BM), -(-geom.L // BN)
    r = ranges.detach().to("cpu")[: BH * nq * 4].view(-1, 4).long()
    x, y, z, w = r.unbind(1)
    ok = (0 <= x) & (x <= y) & (y <= nk) & (0 <= z) & (z <= w) & (w <= nk) & ((z == w) | (y <= z))
    if not bool(ok.all()):
        i = int((~ok).nonzero()[0])
        raise ValueError(f"ranges entry {i} = {r[i].tolist()} is not two ordered ranges within {nk} key tiles")
    o = head_order.detach().to("cpu")[:BH].long()
    if not bool((o.sort().values == torch.arange(BH)).all()):
        raise ValueError("head_order is not a permutation of the heads")


def svg_abi_version():
    return _lib().svg_abi_version()


def svg_last_error():
    msg = _lib().svg_last_error()
    return msg.decode() if msg else ""


def svg_tile_config(dtype, d):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib().svg_tile_config(dtype, d, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def svg_sample_rows(geom, count, seed):
    """`count` distinct video rows of `geom` ([T, T + N*F)), uniform without
    replacement and ascending, as a host int32 numpy array (a pure function of
    the geometry, count and seed; the library draws them, see svg.h)."""
    import numpy as np

    rows = np.empty(max(int(count), 0), dtype=np.int32)
    g = geom.c()
    _check(_lib().svg_sample_rows(ctypes.byref(g), int(count), int(seed) & (2**64 - 1),
                                  rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return rows


def svg_workspace_bytes(geom, dtype, n_rows=0, flags=0):
    n = ctypes.c_size_t()
    g = geom.c()
    _check(_lib().svg_workspace_bytes(ctypes.byref(g), dtype, n_rows, flags, ctypes.byref(n)))
    return n.value


def svg_profile_heads(geom, q, k, v, rows, labels, stats, ws, fallback_rel_mse=0.05, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_shape(geom, t, name)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k and v must share strides")
    BH = geom.B * geom.H
    _check_vec(rows, "rows", _t_i32(), 1)
    _check_vec(labels, "labels", _t_i32(), BH)
    _check_vec(stats, "stats", _t_f32(), BH * 3)
    if DEBUG:
        _debug_rows(geom, rows)
    g = geom.c()
    _check(_lib().svg_profile_heads(ctypes.byref(g), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _strides(q),
                                    _ptr(rows), rows.numel(), float(fallback_rel_mse), _ptr(labels), _ptr(stats),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def svg_search_modes(geom, q, k, v, rows, modes_out, stats_out, ws, lam=0.5, eps=1.0, penalty=0, stream=None):
    """Sparse-vDiT offline mode search: modes_out int32[B*H], stats_out
    float[B*H*8] (mse then loss of skip, window, temporal, stripe)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_shape(geom, t, name)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k and v must share strides")
    BH = geom.B * geom.H
    _check_vec(rows, "rows", _t_i32(), 1)
    _check_vec(modes_out, "modes_out", _t_i32(), BH)
    _check_vec(stats_out, "stats_out", _t_f32(), BH * 8)
    if DEBUG:
        _debug_rows(geom, rows)
    g = geom.c()
    _check(_lib().svg_search_modes(ctypes.byref(g), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _strides(q),
                                   _ptr(rows), rows.numel(), float(lam), float(eps), int(penalty), _ptr(modes_out),
                                   _ptr(stats_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def svg_build_blocks(geom, modes, BM, BN, ranges, head_order, stream=None):
    BH = geom.B * geom.H
    _check_vec(modes, "modes", _t_i32(), BH)
    if BM > 0 and BN > 0:
        _check_vec(ranges, "ranges", _t_i32(), BH * -(-geom.L // BM) * 4)
    _check_vec(head_order, "head_order", _t_i32(), BH)
    if DEBUG:
        _debug_modes(geom, modes)
    g = geom.c()
    _check(_lib().svg_build_blocks(ctypes.byref(g), _ptr(modes), BM, BN, _ptr(ranges), _ptr(head_order),
                                   _stream(stream)))


def svg_layout_permute(geom, src, dst, modes=None, inverse=False, stream=None):
    _check_shape(geom, src, "src")
    _check_shape(geom, dst, "dst")
    if src.dtype != dst.dtype:
        raise TypeError("src and dst dtypes differ")
    _check_vec(modes, "modes", _t_i32(), geom.B * geom.H, optional=True)
    if DEBUG and modes is not None:
        _debug_modes(geom, modes)
    g = geom.c()
    _check(_lib().svg_layout_permute(ctypes.byref(g), _dtype_code(src), _ptr(src), _strides(src), _ptr(dst),
                                     _strides(dst), _ptr(modes), 1 if inverse else 0, _stream(stream)))


def svg_sparse_attention(geom, q, k, v, o, modes, ranges, head_order, qp=None, kp=None, vp=None, op=None,
                         flags=0, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_shape(geom, t, name)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k and v must share strides")
    if kp is not None and (vp is None or vp.stride() != kp.stride()):
        raise ValueError("kp and vp must both be given and share strides")
    if qp is not None and (kp is None or qp.stride() != kp.stride()):
        raise ValueError("qp needs kp and vp with the same strides")
    din = _dtype_code(q)
    BM, BN = svg_tile_config(din, geom.d)
    _check_tile_args(geom, BM, BN, modes, ranges, head_order)
    g = geom.c()
    _check(_lib().svg_sparse_attention(
        ctypes.byref(g), din, _dtype_code(o), _ptr(q), _ptr(k), _ptr(v), _strides(q), _ptr(qp), _ptr(kp), _ptr(vp),
        _strides(kp), _ptr(o), _strides(o), _ptr(op), _strides(op), _ptr(modes), _ptr(ranges), _ptr(head_order),
        BM, BN, flags, _stream(stream)))


def svg_quantize_qk(geom, q, k, modes, q8, sq, k8, sk, stream=None):
    """FP8 E4M3 quantisation of Q (per row) and K (per 64-key tile of the
    working layout): q8, k8 uint8 [B*H*L*d]; sq float32 [B*H*L]; sk float32
    [B*H*ceil(L/64)]."""
    _check_shape(geom, q, "q")
    _check_shape(geom, k, "k")
    if k.stride() != q.stride():
        raise ValueError("q and k must share strides")
    _check_vec(modes, "modes", _t_i32(), geom.B * geom.H)
    if DEBUG:
        _debug_modes(geom, modes)
    g = geom.c()
    _check(_lib().svg_quantize_qk(ctypes.byref(g), _dtype_code(q), _ptr(q), _ptr(k), _strides(q), _ptr(modes),
                                  _ptr(q8), _ptr(sq), _ptr(k8), _ptr(sk), _stream(stream)))


def svg_sparse_attention_fp8(geom, q8, sq, k8, sk, v, o, modes, ranges, head_order, stream=None):
    _check_shape(geom, v, "v")
    _check_shape(geom, o, "o")
    BM, BN = svg_tile_config(BF16, geom.d)
    _check_tile_args(geom, BM, BN, modes, ranges, head_order)
    g = geom.c()
    _check(_lib().svg_sparse_attention_fp8(ctypes.byref(g), _dtype_code(o), _ptr(q8), _ptr(sq), _ptr(k8), _ptr(sk),
                                           _ptr(v), _strides(v), _ptr(o), _strides(o), _ptr(modes), _ptr(ranges),
                                           _ptr(head_order), BM, BN, _stream(stream)))


def svg_quantize_v(geom, v, modes, v8, sv, stream=None):
    """FP8 E4M3 quantisation of V with one scale per head, stored per 64-key
    tile of the working layout, transposed: v8 uint8 [B*H*ceil(L/64)*d*64];
    sv float32 [B*H]."""
    _check_shape(geom, v, "v")
    _check_vec(modes, "modes", _t_i32(), geom.B * geom.H)
    if DEBUG:
        _debug_modes(geom, modes)
    g = geom.c()
    _check(_lib().svg_quantize_v(ctypes.byref(g), _dtype_code(v), _ptr(v), _strides(v), _ptr(modes), _ptr(v8),
                                 _ptr(sv), _stream(stream)))


def svg_sparse_attention_fp8_pv(geom, q8, sq, k8, sk, v8, sv, o, modes, ranges, head_order, stream=None):
    _check_shape(geom, o, "o")
    BM, BN = svg_tile_config(BF16, geom.d)
    _check_tile_args(geom, BM, BN, modes, ranges, head_order)
    g = geom.c()
    _check(_lib().svg_sparse_attention_fp8_pv(ctypes.byref(g), _dtype_code(o), _ptr(q8), _ptr(sq), _ptr(k8),
                                              _ptr(sk), _ptr(v8), _ptr(sv), _ptr(o), _strides(o), _ptr(modes),
                                              _ptr(ranges), _ptr(head_order), BM, BN, _stream(stream)))


def svg_layer_forward(geom, q, k, v, o, ws, rows=None, labels_out=None, stats_out=None, modes_in=None,
                      fallback_rel_mse=0.05, flags=0, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_shape(geom, t, name)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k and v must share strides")
    BH = geom.B * geom.H
    _check_vec(rows, "rows", _t_i32(), 1, optional=True)
    _check_vec(modes_in, "modes_in", _t_i32(), BH, optional=True)
    _check_vec(labels_out, "labels_out", _t_i32(), BH, optional=True)
    _check_vec(stats_out, "stats_out", _t_f32(), BH * 3, optional=True)
    if DEBUG:
        if rows is not None:
            _debug_rows(geom, rows)
        if modes_in is not None:
            _debug_modes(geom, modes_in)
    g = geom.c()
    n_rows = 0 if rows is None else rows.numel()
    _check(_lib().svg_layer_forward(
        ctypes.byref(g), _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v), _strides(q), _ptr(o),
        _strides(o), _ptr(rows), n_rows, float(fallback_rel_mse), _ptr(modes_in), _ptr(labels_out),
        _ptr(stats_out), flags, _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def svg_layer_forward_noalloc(geom, q, k, v, o, rows=None, labels_out=None, stats_out=None, modes_in=None,
                              fallback_rel_mse=0.05, flags=0, stream=None):
    """svg_layer_forward without a workspace argument: the library's fixed
    per-device scratch is used instead (no allocation anywhere in the call;
    calls that overlap on one device race on that scratch)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_shape(geom, t, name)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k and v must share strides")
    BH = geom.B * geom.H
    _check_vec(rows, "rows", _t_i32(), 1, optional=True)
    _check_vec(modes_in, "modes_in", _t_i32(), BH, optional=True)
    _check_vec(labels_out, "labels_out", _t_i32(), BH, optional=True)
    _check_vec(stats_out, "stats_out", _t_f32(), BH * 3, optional=True)
    if DEBUG:
        if rows is not None:
            _debug_rows(geom, rows)
        if modes_in is not None:
            _debug_modes(geom, modes_in)
    g = geom.c()
    n_rows = 0 if rows is None else rows.numel()
    _check(_lib().svg_layer_forward_noalloc(
        ctypes.byref(g), _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v), _strides(q), _ptr(o),
        _strides(o), _ptr(rows), n_rows, float(fallback_rel_mse), _ptr(modes_in), _ptr(labels_out),
        _ptr(stats_out), flags, _stream(stream)))


def svg_noalloc_scratch_bytes():
    """Bytes of the fixed per-device scratch of svg_layer_forward_noalloc."""
    return int(_lib().svg_noalloc_scratch_bytes())


def svg2_workspace_bytes(geom, params):
    n = ctypes.c_size_t()
    g, p = geom.c(), params.c()
    _check(_lib().svg2_workspace_bytes(ctypes.byref(g), ctypes.byref(p), ctypes.byref(n)))
    return n.value


def svg2_kmeans(geom, x, C, iters, mu, labels, perm, start, ws, flags=0, stream=None):
    """k-means of one [B, H, L, d] bf16 tensor per head; mu float32
    [B*H*C*d] (initial centroids with SVG2_INIT_GIVEN), labels / perm int32
    [B*H*L], start int32 [B*H*(C+1)]."""
    _check_shape(geom, x, "x")
    g = geom.c()
    _check(_lib().svg2_kmeans(ctypes.byref(g), _dtype_code(x), _ptr(x), _strides(x), int(C), int(iters), int(flags),
                              _ptr(mu), _ptr(labels), _ptr(perm), _ptr(start), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))


def svg2_forward(geom, params, q, k, v, o, mu_q, mu_k, ws, sel=None, flags=0, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_shape(geom, t, name)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k and v must share strides")
    g, p = geom.c(), params.c()
    _check(_lib().svg2_forward(ctypes.byref(g), ctypes.byref(p), _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k),
                               _ptr(v), _strides(q), _ptr(o), _strides(o), int(flags), _ptr(mu_q), _ptr(mu_k),
                               _ptr(sel), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def alloc_workspace(geom, dtype, n_rows=0, flags=0, device="cuda"):
    """Workspace tensor (uint8, 256-byte aligned by the caching allocator)."""
    import torch
    n = svg_workspace_bytes(geom, dtype, n_rows, flags)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def default_scale(d):
    return 1.0 / math.sqrt(d)
