"""FP8 mode of the oracle: the quantisation the fp8-score attention applies
to Q and K, and attention on the quantised values.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py); shares no code with the
GPU library.

The pages only report that the Sparse-vDiT method composes with FP8
("Sparse-vDiT" review: the appendix lifts the Wan2.1 speedup with FP8); the
scheme is therefore a reading, stated here and in the design notes:
  - the scores Q K^T use FP8 E4M3 (OCP "fn" variant: 1 sign, 4 exponent bits
    with bias 7, 3 mantissa bits, no infinities, max finite 448, code 0x7F /
    0xFF is NaN, subnormals m/8 * 2^-6); P and V stay bf16;
  - every scale is a power of two, so dividing by it is exact and the only
    rounding is the conversion to E4M3 (round to nearest, ties to even);
  - Q: one scale per token row; K: one scale per tile of 64 rows of the
    head's working layout (token-major for TEMPORAL heads); the scale is the
    smallest power of two s with 448 * s >= max |x| (s = 1 for an all-zero
    group), so every scaled value lies in [-448, 448];
  - with FP8 P.V as well: V with one scale per head (the same rule over the
    whole head), and the attention weights in E4M3.  The weights' rounding
    depends on the kernel's running reference max, so no plain oracle
    reproduces it; the oracle for that mode is the exact softmax on the
    dequantised Q, K, V, and the tests bound the weights' rounding
    analytically from the oracle's own weights.
"""
import numpy as np

E4M3_MAX = 448.0
KEY_TILE = 64


def e4m3_decode(codes):
    """float64 values of E4M3FN codes (uint8 array); NaN for 0x7F / 0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite values in code order (codes 0x00 .. 0x7E)
_POS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(x):
    """E4M3FN codes of float64 values with |x| <= 448: round to nearest,
    ties to the even code (even mantissa), sign kept (also for zero)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("value outside the E4M3 range")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)  # first value >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _POS[hi], hi, np.where(pick_hi, hi, lo))
    return (code | np.where(np.signbit(x), 128, 0)).astype(np.uint8)


def pow2_scale(amax):
    """Smallest power of two s with 448 * s >= amax (1 when amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    k = int(np.frexp(amax)[1]) - 10  # 448 * 2^k < amax for this k
    while E4M3_MAX * 2.0 ** k < amax:
        k += 1
    return 2.0 ** k


def quantize_rows(x):
    """Per-row quantisation of [L, d]: (codes uint8 [L, d], scales float64 [L])."""
    x = np.asarray(x, dtype=np.float64)
    s = np.array([pow2_scale(np.max(np.abs(r))) for r in x])
    return e4m3_encode(x / s[:, None]), s


def quantize_tiles(x, tile=KEY_TILE):
    """Per-tile quantisation of [L, d] in tiles of `tile` rows (last ragged):
    (codes uint8 [L, d], scales float64 [ceil(L / tile)])."""
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[0]
    nt = -(-L // tile)
    s = np.array([pow2_scale(np.max(np.abs(x[t * tile:(t + 1) * tile]))) for t in range(nt)])
    rs = np.repeat(s, tile)[:L]
    return e4m3_encode(x / rs[:, None]), s


def dequant_rows(codes, s):
    return e4m3_decode(codes) * np.asarray(s)[:, None]


def dequant_tiles(codes, s, tile=KEY_TILE):
    L = codes.shape[0]
    return e4m3_decode(codes) * np.repeat(np.asarray(s), tile)[:L, None]


def quantize_head(x):
    """One scale for a whole [L, d] group: (codes uint8 [L, d], scale)."""
    x = np.asarray(x, dtype=np.float64)
    s = pow2_scale(np.max(np.abs(x)) if x.size else 0.0)
    return e4m3_encode(x / s), s
