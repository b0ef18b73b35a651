"""Seeded synthetic inputs for the sparse-attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no masks, no attention, no classification), so both the
GPU tests and the CPU oracle can take their inputs from it.

Workloads are shaped like the video models the pages evaluate on (CogVideoX,
HunyuanVideo, Wan2.1): N frames of F tokens, H heads of width d, optional text
prefix.  There are no model activations here, so query/key rows are planted:
a head of a given kind shares a per-frame vector (spatial-like), a
per-position vector (temporal-like) or a global vector (stripe-like) between
its queries and keys, plus independent Gaussian noise; values are iid N(0,1).

Random-number recipe (numpy PCG64, fixed draw order), seed = 1000*config + call:
  head kinds / modes (when drawn) from default_rng(seed);
  head h from its own stream default_rng([seed, h + 1]): planted vectors,
  then query noise [L, d], key noise [L, d], values [L, d];
  sampled rows from default_rng(seed + 500).
Values are rounded to bf16 (round-to-nearest-even) for the bf16 workloads;
both sides receive the same bits.
"""
import math

import numpy as np

# head kinds / modes; numbering equals the library's mode enum
SPATIAL, TEMPORAL, FULL, SKIP, WINDOW, STRIPE = range(6)
UNSTRUCTURED = FULL  # an unstructured head carries no planted signal

# the synthetic workloads (shapes of the pages' models), by index and name
TINY_FP32, COGVIDEOX, HUNYUANVIDEO, HUNYUANVIDEO_TEXT, SPARSE_VDIT = range(5)
WORKLOADS = {
    0: dict(name="tiny-fp32 4x64 h2 d64", N=4, F=64, T=0, H=2, d=64, a1=1, a2=8, dtype="f32",
            signal=3.0, noise=0.3, sample="all"),
    1: dict(name="cogvideox-like 13x4080 h48 d64", N=13, F=4080, T=0, H=48, d=64, a1=2, a2=170,
            dtype="bf16", signal=1.5, noise=1.0, sample=0.01),
    2: dict(name="hunyuanvideo-like 33x3600 h24 d128", N=33, F=3600, T=0, H=24, d=128, a1=2, a2=160,
            dtype="bf16", signal=1.5, noise=1.0, sample=0.01),
    3: dict(name="hunyuanvideo-like + 256 text, mixed heads", N=33, F=3600, T=256, H=24, d=128, a1=2,
            a2=160, dtype="bf16", signal=1.5, noise=1.0, sample=0.01),
    4: dict(name="sparse-vdit pattern set 21x1560 h40 d128", N=21, F=1560, T=0, H=40, d=128, a1=2,
            a2=128, window=1560, stripe=512, dtype="bf16", signal=1.5, noise=1.0, sample=None),
}


def bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sample_rows(N, F, T, frac, seed):
    """ceil(frac * N*F) distinct video rows, uniform without replacement, sorted."""
    n_vid = N * F
    if frac == "all":
        return np.arange(T, T + n_vid, dtype=np.int32)
    n = max(1, math.ceil(frac * n_vid))
    rng = np.random.default_rng(seed)
    rows = rng.choice(n_vid, size=n, replace=False)
    return (np.sort(rows) + T).astype(np.int32)


def head_kinds(cfg, rng):
    c = WORKLOADS[cfg]
    H = c["H"]
    if cfg == 0:
        return np.array([SPATIAL, TEMPORAL], dtype=np.int32)
    if cfg == 1:
        return np.array([SPATIAL if h % 2 == 0 else TEMPORAL for h in range(H)], dtype=np.int32)
    if cfg == 2:
        return np.where(rng.random(H) < 0.5, SPATIAL, TEMPORAL).astype(np.int32)
    if cfg == 3:
        # 40 % / 40 % / 20 % of 24 heads by largest remainder: 10 / 9 / 5
        kinds = np.array([SPATIAL] * 10 + [TEMPORAL] * 9 + [UNSTRUCTURED] * 5, dtype=np.int32)
        return kinds[rng.permutation(H)]
    if cfg == 4:
        per = H // 5
        kinds = np.array([FULL, SKIP, WINDOW, TEMPORAL, STRIPE] * per, dtype=np.int32)
        return kinds[rng.permutation(H)]
    raise ValueError(cfg)


def _plant(kind, cfg, c, rng, L):
    """Planted signal rows [L, d] (float32) for one head; zeros if none."""
    N, F, T, d, s = c["N"], c["F"], c["T"], c["d"], c["signal"]
    sig_q = np.zeros((L, d), dtype=np.float32)
    sig_k = np.zeros((L, d), dtype=np.float32)
    vid = slice(T, T + N * F)
    if kind in (SPATIAL, WINDOW):  # per-frame vector e_i
        e = rng.standard_normal((N, d), dtype=np.float32)
        rows = np.repeat(e, F, axis=0) * s
        sig_q[vid] = rows
        sig_k[vid] = rows
    elif kind == TEMPORAL:  # per-position vector p_j
        p = rng.standard_normal((F, d), dtype=np.float32)
        rows = np.tile(p, (N, 1)) * s
        sig_q[vid] = rows
        sig_k[vid] = rows
    elif kind == STRIPE:  # shared vector in every query and in the first keys
        u = rng.standard_normal((1, d), dtype=np.float32) * s
        sig_q[vid] = u
        n_str = min(c.get("stripe", 512), N * F)
        sig_k[T:T + n_str] = u
    return sig_q, sig_k


def _head(cfg, c, kind, seed, h, L):
    rng = np.random.default_rng([seed, h + 1])
    sig_q, sig_k = _plant(kind, cfg, c, rng, L)
    d = c["d"]
    q = sig_q + c["noise"] * rng.standard_normal((L, d), dtype=np.float32)
    k = sig_k + c["noise"] * rng.standard_normal((L, d), dtype=np.float32)
    v = rng.standard_normal((L, d), dtype=np.float32)
    if c["dtype"] == "bf16":
        q, k, v = (bf16_to_f32(bf16_bits(a)) for a in (q, k, v))
    return q, k, v


def make_inputs(cfg, call=0, heads=None, workers=8):
    """Inputs of one workload call.

    Returns dict with q, k, v as float32 arrays [len(heads), L, d] holding
    exactly the values both sides use (bf16-representable for bf16
    workloads), the head kinds of all heads, the sampled rows, the seed and
    the config dict.  ``heads`` selects which heads are materialised (every
    head has its own random stream, so a subset is drawn identically).
    """
    import concurrent.futures
    c = WORKLOADS[cfg]
    N, F, T, H, d = c["N"], c["F"], c["T"], c["H"], c["d"]
    L = T + N * F
    seed = 1000 * cfg + call
    kinds = head_kinds(cfg, np.random.default_rng(seed))
    keep = list(range(H)) if heads is None else list(heads)
    q = np.empty((len(keep), L, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def fill(i):
        q[i], k[i], v[i] = _head(cfg, c, kinds[keep[i]], seed, keep[i], L)

    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(len(keep))))
    rows = None
    if c["sample"] is not None:
        rows = sample_rows(N, F, T, c["sample"], seed + 500)
    return dict(q=q, k=k, v=v, kinds=kinds, rows=rows, seed=seed, cfg=c, heads=keep)


def small_config(N, F, T, H, d, a1, a2, kinds, seed, signal=1.5, noise=1.0, dtype="bf16",
                 window=None, stripe=512):
    """Inputs for an ad-hoc scaled-down shape with explicit head kinds."""
    c = dict(N=N, F=F, T=T, H=H, d=d, a1=a1, a2=a2, signal=signal, noise=noise, dtype=dtype,
             window=window if window is not None else F, stripe=stripe)
    L = T + N * F
    rng = np.random.default_rng(seed)
    q = np.empty((H, L, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    for h in range(H):
        sig_q, sig_k = _plant(int(kinds[h]), None, c, rng, L)
        q[h] = sig_q + noise * rng.standard_normal((L, d), dtype=np.float32)
        k[h] = sig_k + noise * rng.standard_normal((L, d), dtype=np.float32)
        v[h] = rng.standard_normal((L, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = (bf16_to_f32(bf16_bits(a)) for a in (q, k, v))
    return dict(q=q, k=k, v=v, kinds=np.asarray(kinds, dtype=np.int32), cfg=c)


def svg2_inputs(N, F, T, H, d, G, seed, spread=1.0, noise=0.3, dtype="bf16"):
    """Inputs for the SVG2 path: per head, G semantic groups with centres
    ~ N(0, spread^2) in d dimensions; every token belongs to a group drawn
    uniformly at random (groups are scattered over positions, not frames);
    its query and key are the group centre plus independent N(0, noise^2)
    noise, its value iid N(0, 1).  Draw order per head (own stream
    default_rng([seed, h + 1])): centres, groups, q-noise, k-noise, v."""
    L = T + N * F
    q = np.empty((H, L, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    groups = np.empty((H, L), dtype=np.int64)
    centres = np.empty((H, G, d), dtype=np.float32)
    for h in range(H):
        rng = np.random.default_rng([seed, h + 1])
        c = rng.standard_normal((G, d), dtype=np.float32) * spread
        g = rng.integers(0, G, L)
        q[h] = c[g] + noise * rng.standard_normal((L, d), dtype=np.float32)
        k[h] = c[g] + noise * rng.standard_normal((L, d), dtype=np.float32)
        v[h] = rng.standard_normal((L, d), dtype=np.float32)
        groups[h], centres[h] = g, c
    if dtype == "bf16":
        q, k, v = (bf16_to_f32(bf16_bits(a)) for a in (q, k, v))
    return dict(q=q, k=k, v=v, groups=groups, centres=centres)
