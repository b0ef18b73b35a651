"""Shared helpers of the GPU parity tests (marshalling only, no method
arithmetic): upload seeded inputs, run the library, compare with the oracle."""
import numpy as np

import oracle
import sparse_attention_video_svg_amd as svg

# Tolerances for attention outputs (bf16 inputs, fp32 accumulation) and for
# the fp32 end-to-end path.
BF16_MAX_ABS, BF16_RMS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5


def to_device(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def ogeom(g):
    """Oracle geometry from a library geometry."""
    return oracle.geom(g.N, g.F, g.T, g.a1, g.a2, g.window, g.stripe)


def scale_of(g):
    return g.scale if g.scale > 0 else 1.0 / np.sqrt(g.d)


def check_close(got, ref, dtype_name, what=""):
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    mx = float(err.max()) if err.size else 0.0
    rms = float(np.sqrt((err ** 2).mean())) if err.size else 0.0
    if dtype_name == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max-abs {mx:.3e} > {F32_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max-abs {mx:.3e} > {BF16_MAX_ABS}"
        assert rms <= BF16_RMS, f"{what}: rms {rms:.3e} > {BF16_RMS}"
    return mx, rms


def block_bitmap_from_ranges(ranges_np, nq, nk):
    """Expand the library's per-query-tile key-tile ranges into a bitmap."""
    bm = np.zeros((nq, nk), dtype=np.uint8)
    r = ranges_np.reshape(nq, 4)
    for qb in range(nq):
        s1, e1, s2, e2 = r[qb]
        assert 0 <= s1 <= e1 <= nk and 0 <= s2 <= e2 <= nk
        assert e1 <= s2 or s2 == e2, "ranges must be sorted and disjoint"
        bm[qb, s1:e1] = 1
        bm[qb, s2:e2] = 1
    return bm


def sample_check_rows(L, T, extra=(), n=48, seed=0):
    """Rows to compare at full size: first/last rows, text boundary, seeded picks."""
    rng = np.random.default_rng(seed)
    rows = {0, L - 1, max(0, T - 1), T, min(L - 1, T + 1)} | set(int(x) for x in extra if 0 <= x < L)
    rows |= set(rng.choice(L, size=min(n, L), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def rows_per_tile(L, BM, seed=0):
    """One seeded row inside every BM-row query tile (the last tile may be
    ragged), so a full-size check visits every tile of the kernel's grid."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, L, BM)
    ends = np.minimum(starts + BM, L)
    return (starts + (rng.random(starts.size) * (ends - starts)).astype(np.int64)).astype(np.int64)
