"""Pins for the oracle's MXFP4 coding (CPU only).

The oracle codes a value by searching the E2M1 grid for the nearest point. These
tests check it against numpy's own half-to-even rounding applied binade by binade
(E2M1 has a step of 0.5 below 2, 1 in [2, 4) and 2 in [4, 8)), exhaustively over
every finite bf16 bit pattern and a window of block exponents, and check the
block-exponent rule against numpy's frexp.
"""

import numpy as np
import pytest

from oracle import (E2M1_GRID, block_scale_exponent, decode_e2m1, floor_log2_f32,
                    mxfp4_quantize, quantize_e2m1, quantize_weight_ref, unpack_nibbles)
from synth import bf16_to_f32

VALUE_TO_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def independent_code(v):
    """E2M1 code by binade-wise np.round (half to even) and saturation at 6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    q = np.where(a < 2, np.round(a * 2) / 2,
                 np.where(a < 4, np.round(a), 2 * np.round(a / 2)))
    q = np.minimum(q, 6.0)
    lut = np.zeros(13, dtype=np.uint8)
    for val, code in VALUE_TO_CODE.items():
        lut[int(val * 2)] = code
    codes = lut[(q * 2).astype(np.int64)]
    return codes | (np.signbit(v).astype(np.uint8) << 3)


def all_finite_bf16():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(u)
    keep = np.isfinite(f)
    return u[keep], f[keep]


def test_grid_points_and_midpoints():
    for c in range(16):
        v = decode_e2m1(np.array([c], np.uint8))
        back = quantize_e2m1(v)[0]
        # -0 and +0 keep their sign bit, so every code round-trips
        if c == 8:
            v = np.array([-0.0])
            back = quantize_e2m1(v)[0]
        assert back == c
    # every midpoint goes to the even code
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in mids.items():
        assert quantize_e2m1(np.array([v]))[0] == c
        assert quantize_e2m1(np.array([-v]))[0] == c | 8
    # saturation
    assert quantize_e2m1(np.array([6.5, 7.0, 7.99, 1e30]))[:].tolist() == [7, 7, 7, 7]
    # just above / below midpoints
    eps = 2.0 ** -40
    assert quantize_e2m1(np.array([0.25 + eps]))[0] == 1
    assert quantize_e2m1(np.array([0.75 - eps]))[0] == 1
    assert quantize_e2m1(np.array([5.0 + eps]))[0] == 7


def test_quantizer_exhaustive_bf16_times_exponents():
    u, f = all_finite_bf16()
    f = f.astype(np.float64)
    # exponents centred on each value's own block exponent (so |v| spans (0, 16)),
    # plus fixed exponents at and near the clamp edges
    nz = np.abs(f) > 0
    base = np.where(nz, block_scale_exponent(np.abs(f).astype(np.float32)), 0)
    vs = []
    for d in range(-2, 5):
        vs.append(f * np.ldexp(1.0, -(base + d)))
    for e in (-127, -126, -120, 0, 1, 100, 127):
        vs.append(f * np.ldexp(1.0, -e))
    v = np.concatenate(vs)
    v = v[np.isfinite(v)]
    assert np.array_equal(quantize_e2m1(v), independent_code(v))


def test_quantizer_monotone_in_magnitude():
    v = np.linspace(0, 9, 100001)
    c = quantize_e2m1(v)
    assert np.all(np.diff(decode_e2m1(c)) >= 0)


def test_floor_log2_against_frexp():
    u, f = all_finite_bf16()
    pos = f > 0
    rng = np.random.default_rng(5)
    bits = rng.integers(1, 0x7F800000, size=200000, dtype=np.uint32)
    extra = bits.view(np.float32)
    sub = np.arange(1, 1 << 12, dtype=np.uint32).view(np.float32)  # smallest subnormals
    topsub = (np.uint32(0x007FFFFF) - np.arange(4096, dtype=np.uint32)).view(np.float32)
    a = np.concatenate([f[pos], extra, sub, topsub])
    _, ex = np.frexp(a.astype(np.float64))
    assert np.array_equal(floor_log2_f32(a), ex - 1)


def test_block_exponent_rule():
    rng = np.random.default_rng(9)
    a = np.abs(rng.standard_normal(100000) * np.exp(rng.uniform(-80, 80, 100000))).astype(np.float32)
    a = a[(a > 0) & np.isfinite(a)]
    e = block_scale_exponent(a)
    inner = (e > -127) & (e < 127)
    lo = np.ldexp(1.0, e + 2)
    hi = np.ldexp(1.0, e + 3)
    assert np.all((lo[inner] <= a[inner]) & (a[inner] < hi[inner]))
    assert block_scale_exponent(np.array([0.0], np.float32))[0] == -127
    # tiny blocks clamp at -127 (byte 0x00); the largest finite float32 gives 125
    assert block_scale_exponent(np.array([2.0 ** -126], np.float32))[0] == -127
    assert block_scale_exponent(np.array([2.0 ** -124], np.float32))[0] == -126
    assert block_scale_exponent(np.array([np.finfo(np.float32).max], np.float32))[0] == 125


def test_block_max_code_is_4_or_6():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((50, 320)) * rng.lognormal(0, 3, (50, 1))).astype(np.float32)
    codes, e = mxfp4_quantize(x)
    mags = (codes & 7).reshape(50, 10, 32).max(-1)
    assert set(np.unique(mags)) <= {6, 7}


def test_weight_quantizer_matches_independent_rule():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for a test input
    codes_p, scales = quantize_weight_ref(wb)
    codes = unpack_nibbles(codes_p)
    w32 = bf16_to_f32(wb).astype(np.float64)
    e = scales.astype(np.int64) - 127
    for t in range(8):
        for b in range(4):
            blk = w32[t, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            _, ex = np.frexp(amax)
            assert e[t, b] == ex - 1 - 2
            v = blk / 2.0 ** e[t, b]
            assert np.array_equal(codes[t, 32 * b:32 * b + 32], independent_code(v))


@pytest.mark.parametrize("c", range(16))
def test_decode_table(c):
    val = decode_e2m1(np.array([c], np.uint8))[0]
    assert abs(val) == E2M1_GRID[c & 7]
    assert np.signbit(val) == bool(c & 8) or (c == 8 and val == 0)
