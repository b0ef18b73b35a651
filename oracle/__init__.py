"""CPU oracle for the Sparse VideoGen sparse-attention path.

TEST INFRASTRUCTURE ONLY: this package may be imported by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``,
never by the product package.  It shares no code with the GPU library.

``svg_oracle.c`` holds the plain fp64 implementation (compiled with gcc into
``libsvg_oracle.so``); ``ref_numpy.py`` is an independent dense numpy
restatement used to cross-check it on tiny shapes.  Each function cites the
passage it follows in its C docstring.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "svg_oracle.c")
LIB = os.path.join(HERE, "libsvg_oracle.so")

SPATIAL, TEMPORAL, FULL, SKIP, WINDOW, STRIPE, TEMPORAL_PERMUTED = range(7)
MODE_NAMES = {SPATIAL: "spatial", TEMPORAL: "temporal", FULL: "full", SKIP: "skip",
              WINDOW: "window", STRIPE: "stripe", TEMPORAL_PERMUTED: "temporal_permuted"}


def build():
    """Compile the oracle with gcc (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)


class OgGeom(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("F", ctypes.c_int32), ("T", ctypes.c_int32),
                ("a1", ctypes.c_int32), ("a2", ctypes.c_int32), ("window", ctypes.c_int32),
                ("stripe", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.POINTER
        g = P(OgGeom)
        vp = ctypes.c_void_p
        L.og_perm.argtypes = [g, ctypes.c_int64]
        L.og_perm.restype = ctypes.c_int64
        L.og_perm_inv.argtypes = [g, ctypes.c_int64]
        L.og_perm_inv.restype = ctypes.c_int64
        L.og_mask.argtypes = [g, ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
        L.og_mask.restype = ctypes.c_int
        L.og_permute_rows.argtypes = [g, ctypes.c_int64, vp, vp, ctypes.c_int]
        L.og_permute_rows.restype = None
        L.og_row_intervals.argtypes = [g, ctypes.c_int, ctypes.c_int64, vp, vp, ctypes.c_int]
        L.og_row_intervals.restype = ctypes.c_int
        L.og_max_intervals.argtypes = [g]
        L.og_max_intervals.restype = ctypes.c_int
        L.og_attention_brute.argtypes = [g, ctypes.c_int, ctypes.c_int32, ctypes.c_double, vp, vp, vp, vp]
        L.og_attention_brute.restype = None
        L.og_attention_rows.argtypes = [g, ctypes.c_int, ctypes.c_int32, ctypes.c_double, vp, vp, vp,
                                        vp, ctypes.c_int64, vp]
        L.og_attention_rows.restype = None
        L.og_profile_head.argtypes = [g, ctypes.c_int32, ctypes.c_double, vp, vp, vp, vp, ctypes.c_int64,
                                      ctypes.c_double, vp, vp]
        L.og_profile_head.restype = None
        L.og_mask_nnz.argtypes = [g, ctypes.c_int]
        L.og_mask_nnz.restype = ctypes.c_int64
        L.og_search_head.argtypes = [g, ctypes.c_int32, ctypes.c_double, vp, vp, vp, vp, ctypes.c_int64,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_int, vp, vp, vp, vp]
        L.og_search_head.restype = None
        L.og_blocks_brute.argtypes = [g, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, vp]
        L.og_blocks_brute.restype = None
        L.og_blocks_rows.argtypes = [g, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, vp]
        L.og_blocks_rows.restype = None
        L.og_head_order.argtypes = [ctypes.c_int32, vp, vp]
        L.og_head_order.restype = None
        L.og_num_threads.argtypes = []
        L.og_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def geom(N, F, T=0, a1=1, a2=1, window=1, stripe=1):
    return OgGeom(N, F, T, a1, a2, window, stripe)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def ltot(g):
    return g.T + g.N * g.F


def perm_index(g):
    """pi as an int64 array: pi[x] = token-major index of natural token x."""
    L = lib()
    return np.array([L.og_perm(ctypes.byref(g), x) for x in range(ltot(g))], dtype=np.int64)


def perm_inv_index(g):
    L = lib()
    return np.array([L.og_perm_inv(ctypes.byref(g), x) for x in range(ltot(g))], dtype=np.int64)


def mask(g, mode, x1, x2):
    return lib().og_mask(ctypes.byref(g), mode, x1, x2)


def mask_matrix(g, mode):
    """Dense [L, L] uint8 mask through the C predicate (tiny shapes)."""
    L = ltot(g)
    Lb = lib()
    m = np.zeros((L, L), dtype=np.uint8)
    gb = ctypes.byref(g)
    for x1 in range(L):
        for x2 in range(L):
            m[x1, x2] = Lb.og_mask(gb, mode, x1, x2)
    return m


def permute_rows(g, src, inverse=False):
    """Row permutation of a [L, ...] array (any dtype), forward or inverse."""
    src = np.ascontiguousarray(src)
    dst = np.empty_like(src)
    row_bytes = src.strides[0]
    lib().og_permute_rows(ctypes.byref(g), row_bytes, _ptr(src), _ptr(dst), int(bool(inverse)))
    return dst


def max_intervals(g):
    """Most intervals one row can have (text columns + one per frame)."""
    return int(lib().og_max_intervals(ctypes.byref(g)))


def row_intervals(g, mode, x1, max_n=None):
    """Active keys of row x1 as [(lo, hi), ...]; raises if more than max_n
    intervals would be needed (default: enough for any row)."""
    if max_n is None:
        max_n = max_intervals(g)
    lo = np.zeros(max(max_n, 1), dtype=np.int64)
    hi = np.zeros(max(max_n, 1), dtype=np.int64)
    n = lib().og_row_intervals(ctypes.byref(g), mode, x1, _ptr(lo), _ptr(hi), max_n)
    if n < 0:
        raise ValueError(f"row {x1} of mode {mode} needs more than {max_n} intervals")
    return list(zip(lo[:n].tolist(), hi[:n].tolist()))


def attention_brute(g, mode, q, k, v, scale):
    q, k, v = _f32(q), _f32(k), _f32(v)
    L, d = q.shape
    out = np.zeros((L, d), dtype=np.float64)
    lib().og_attention_brute(ctypes.byref(g), mode, d, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(out))
    return out


def attention_rows(g, mode, q, k, v, scale, rows):
    q, k, v = _f32(q), _f32(k), _f32(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    d = q.shape[1]
    out = np.zeros((rows.shape[0], d), dtype=np.float64)
    lib().og_attention_rows(ctypes.byref(g), mode, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(rows), rows.shape[0], _ptr(out))
    return out


def profile_head(g, q, k, v, scale, rows, fallback=0.05):
    """Returns (label, stats[3] = rel_spatial, rel_temporal, mean O_full^2)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    stats = np.zeros(3, dtype=np.float64)
    label = np.zeros(1, dtype=np.int32)
    lib().og_profile_head(ctypes.byref(g), q.shape[1], float(scale), _ptr(q), _ptr(k), _ptr(v),
                          _ptr(rows), rows.shape[0], float(fallback), _ptr(stats), _ptr(label))
    return int(label[0]), stats


def mask_nnz(g, mode):
    """Active (query, key) pairs of a mask over the whole map."""
    return int(lib().og_mask_nnz(ctypes.byref(g), mode))


SEARCH_CANDIDATES = (SKIP, WINDOW, TEMPORAL, STRIPE)


def search_head(g, q, k, v, scale, rows, lam=0.5, eps=1.0, penalty=0):
    """Sparse-vDiT mode search of one head.  Returns (mode, mse[4], loss[4],
    sparsity[4]) with the candidates in SEARCH_CANDIDATES order."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    mse, loss, sp = (np.zeros(4, dtype=np.float64) for _ in range(3))
    mode = np.zeros(1, dtype=np.int32)
    lib().og_search_head(ctypes.byref(g), q.shape[1], float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(rows),
                         rows.shape[0], float(lam), float(eps), int(penalty), _ptr(mse), _ptr(loss), _ptr(sp),
                         _ptr(mode))
    return int(mode[0]), mse, loss, sp


def blocks(g, mode, BM, BN, brute=False):
    L = ltot(g)
    nq, nk = -(-L // BM), -(-L // BN)
    bm = np.zeros((nq, nk), dtype=np.uint8)
    f = lib().og_blocks_brute if brute else lib().og_blocks_rows
    f(ctypes.byref(g), mode, BM, BN, _ptr(bm))
    return bm


def head_order(work):
    work = np.ascontiguousarray(work, dtype=np.int64)
    order = np.zeros(work.shape[0], dtype=np.int32)
    lib().og_head_order(work.shape[0], _ptr(work), _ptr(order))
    return order


def num_threads():
    return lib().og_num_threads()
