"""Pins of the oracle's FP8 (E4M3FN) quantisation (oracle/fp8.py) against the
format's definition and against an exhaustive nearest-value search: named
codes, monotone decode, exact round trips, ties to even, nearest rounding
checked value by value against all 254 finite values, and the power-of-two
scale rule."""
import math

import numpy as np
import pytest

from oracle import fp8


def test_named_codes():
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
            0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5, 0x77: 240.0, 0x78: 256.0}
    for c, v in want.items():
        assert fp8.e4m3_decode(np.array([c], dtype=np.uint8))[0] == v, hex(c)
    assert math.isnan(fp8.e4m3_decode(np.array([0x7F], dtype=np.uint8))[0])
    assert math.isnan(fp8.e4m3_decode(np.array([0xFF], dtype=np.uint8))[0])
    z = fp8.e4m3_decode(np.array([0x80], dtype=np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0


def test_decode_is_monotone_and_round_trips():
    pos = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(finite)), finite)


def test_ties_go_to_even_codes():
    pos = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    mid = (pos[:-1] + pos[1:]) / 2
    got = fp8.e4m3_encode(mid)
    c = np.arange(126)
    assert np.array_equal(got, np.where(c % 2 == 0, c, c + 1).astype(np.uint8))
    up = fp8.e4m3_encode(np.nextafter(mid, np.inf))
    dn = fp8.e4m3_encode(np.nextafter(mid, -np.inf))
    assert np.array_equal(up, (c + 1).astype(np.uint8)) and np.array_equal(dn, c.astype(np.uint8))


def test_nearest_value_by_exhaustive_search():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 1e-2, 2000), rng.normal(0, 3, 2000)])
    x = np.clip(x, -448, 448)
    codes = fp8.e4m3_encode(x)
    table = fp8.e4m3_decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8))
    got = fp8.e4m3_decode(codes)
    best = np.min(np.abs(table[None, :] - x[:, None]), axis=1)
    assert np.array_equal(np.abs(got - x), best)


@pytest.mark.parametrize("amax,s", [(448.0, 1.0), (449.0, 2.0), (224.0, 0.5), (1.0, 2.0 ** -8), (0.0, 1.0),
                                    (448.0 * 2 ** -20, 2.0 ** -20), (3.0e4, 128.0)])
def test_pow2_scale(amax, s):
    assert fp8.pow2_scale(amax) == s
    if amax > 0:
        assert 224.0 < amax / s <= 448.0


def test_quantize_rows_and_tiles_bounds():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 2, (130, 64)).astype(np.float32).astype(np.float64)
    x[5] = 0.0
    for codes, scales, deq in ((*fp8.quantize_rows(x), None), (*fp8.quantize_tiles(x), None)):
        assert codes.dtype == np.uint8 and codes.shape == x.shape
        assert np.all(np.log2(scales) == np.round(np.log2(scales)))
    c, s = fp8.quantize_rows(x)
    assert s[5] == 1.0 and np.all(c[5] == 0)
    d = fp8.dequant_rows(c, s)
    # error at most half the spacing of E4M3 at the value (relative 2^-4, or
    # the subnormal step 2^-10 * s near zero)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[:, None])
    assert np.all(np.abs(d - x) <= bound)
    c2, s2 = fp8.quantize_tiles(x)
    assert s2.shape == (3,)
    d2 = fp8.dequant_tiles(c2, s2)
    bound2 = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.repeat(s2, 64)[:130, None])
    assert np.all(np.abs(d2 - x) <= bound2)


def test_representable_values_are_unchanged():
    """Values that are already E4M3 numbers times a power-of-two scale come
    back exactly, so fp8 scores equal the bf16 ones on such inputs."""
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 0x7F, (64, 32)).astype(np.uint8) | (rng.integers(0, 2, (64, 32)) * 128).astype(np.uint8)
    codes[:, 0] = 0x7E  # every row holds 448 -> scale exactly 2^-3 after scaling by 2^-3
    x = fp8.e4m3_decode(codes) * 2.0 ** -3
    c, s = fp8.quantize_rows(x)
    assert np.all(s == 2.0 ** -3) and np.array_equal(c, codes)
    assert np.array_equal(fp8.dequant_rows(c, s), x)


def test_quantize_head():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1.5, (200, 64)).astype(np.float32).astype(np.float64)
    c, s = fp8.quantize_head(x)
    assert c.shape == x.shape and c.dtype == np.uint8
    assert 224.0 < np.max(np.abs(x)) / s <= 448.0 and np.log2(s) == np.round(np.log2(s))
    d = fp8.e4m3_decode(c) * s
    assert np.all(np.abs(d - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s))
    z, sz = fp8.quantize_head(np.zeros((5, 8)))
    assert sz == 1.0 and np.all(z == 0)
    # values that are E4M3 numbers times the head's scale come back exactly
    codes = rng.integers(0, 0x7F, (40, 16)).astype(np.uint8)
    codes[3, 3] = 0x7E
    y = fp8.e4m3_decode(codes) * 2.0 ** -5
    cy, sy = fp8.quantize_head(y)
    assert sy == 2.0 ** -5 and np.array_equal(cy, codes)


@pytest.mark.parametrize("spread,n,seed", [(0.5, 300, 0), (4.0, 300, 1), (20.0, 500, 2), (0.05, 4000, 3),
                                           (30.0, 6000, 4)])
def test_fp8_weight_bound_holds_for_emulated_rounding(spread, n, seed):
    """The bound used for the FP8 P.V outputs, checked against the scheme
    emulated here: weights 2^(x - m_ref + 6) rounded to E4M3 by the oracle's
    encoder for references m_ref anywhere in [m - 2, m], with flat rows
    (many keys far below the max) and peaky ones."""
    from fp8_bounds import fp8_pv_bound
    rng = np.random.default_rng(seed)
    x = rng.normal(0, spread, n)
    x[rng.integers(0, n)] += 3 * spread  # one dominant key
    v = rng.normal(0, 1, (n, 16))
    m = x.max()
    w = np.exp2(x - m)
    w /= w.sum()
    o = w @ v
    bound = fp8_pv_bound(x, w, v, o)
    for m_ref in (m, m - 0.5, m - 1.3, m - 2.0):
        p = fp8.e4m3_decode(fp8.e4m3_encode(np.exp2(x - m_ref + 6)))
        o8 = (p @ v) / p.sum()
        assert np.all(np.abs(o8 - o) <= bound + 1e-12), (m_ref, np.max(np.abs(o8 - o) - bound))
