"""Pins of the oracle's RMSNorm absorption (O0): the bf16 rounding of a float32
value by brute force, the row scale against an exactly rounded sum, exact
power-of-two scaling, the fixed summation order on rows built so that other
orders give other bits, and the prepare chain."""

import math

import numpy as np
import pytest

from oracle import (bf16_bits_to_f32, f32_to_bf16_bits_rne, prepare_ref, rms_normalize_ref, rms_row_scale_ref,
                    rms_sum_sq_ref)
from synth import bf16_round


def _bits(vals):
    return bf16_round(np.asarray(vals, dtype=np.float32))


def test_f32_to_bf16_brute_force():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 31, 20000, dtype=np.uint32)  # positive patterns
    u = u[(u >> 23) < 255]  # finite
    u = u[((u >> 23) != 254) | ((u & 0x7FFFFF) < 0x7F0000)]  # stay clear of rounding to inf
    # add exact ties and subnormals
    ties = ((rng.integers(1, 250, 2000, dtype=np.uint32) << 23) | (rng.integers(0, 128, 2000, dtype=np.uint32) << 16)
            | 0x8000)
    subn = rng.integers(1, 0x7FFFFF, 2000, dtype=np.uint32)
    u = np.concatenate([u, ties, subn])
    sign = rng.integers(0, 2, len(u), dtype=np.uint32) << 31
    v = (u | sign).view(np.float32)
    got = f32_to_bf16_bits_rne(v)
    lo = ((u | sign) >> 16).astype(np.uint16)  # truncation toward zero
    hi = (lo + 1).astype(np.uint16)            # next bf16 away from zero
    vl = bf16_bits_to_f32(lo).astype(np.float64)
    vh = bf16_bits_to_f32(hi).astype(np.float64)
    x = v.astype(np.float64)
    dl, dh = np.abs(x - vl), np.abs(vh - x)
    want = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(got, want)
    # values already on the bf16 grid map to themselves
    b = rng.integers(0, 0x7F7F, 5000).astype(np.uint16)
    assert np.array_equal(f32_to_bf16_bits_rne(bf16_bits_to_f32(b)), b)


def test_row_scale_matches_exactly_rounded_sum():
    rng = np.random.default_rng(6)
    for K in (32, 96, 128, 4096, 4128):
        x = _bits(rng.standard_normal((40, K)) * rng.lognormal(0, 2, (40, 1)))
        r = rms_row_scale_ref(x, 1e-5)
        xf = bf16_bits_to_f32(x).astype(np.float64)
        for t in range(x.shape[0]):
            s = math.fsum((xf[t] * xf[t]).tolist())
            want = np.float32(1.0 / math.sqrt(s / K + float(np.float32(1e-5))))
            assert r[t] == want, (K, t)


def test_row_scale_power_of_two_scaling_and_constant_rows():
    rng = np.random.default_rng(7)
    x = _bits(rng.standard_normal((20, 256)))
    tiny = 2.0 ** -149  # vanishes against the mean of these rows
    r = rms_row_scale_ref(x, tiny)
    for k in (-6, -1, 3, 9):
        xs = _bits(bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        assert np.array_equal(rms_row_scale_ref(xs, tiny), (r * np.float32(2.0 ** -k)).astype(np.float32))
    for c in (0.25, 1.0, 8.0):
        row = np.full((1, 64), c, np.float32)
        row[0, ::3] *= -1
        xn, rr = rms_normalize_ref(_bits(row), tiny)
        assert rr[0] == np.float32(1.0 / c)
        assert np.array_equal(bf16_bits_to_f32(xn), np.sign(row).astype(np.float32))


def test_sum_order_is_sequential_in_blocks_then_pairwise():
    # squares: 1 and 2**-54 (x = 2**-27). Within a block the squares are added
    # one after the other: 1 + 2**-54 rounds back to 1 four times, where adding
    # the small ones first would give 1 + 2**-52.
    one, small = 1.0, 2.0 ** -27
    row = np.zeros((1, 32), np.float32)
    row[0, :5] = [one, small, small, small, small]
    assert rms_sum_sq_ref(_bits(row))[0] == 1.0
    # Blocks [1, 0, 2**-53, 2**-53] (each 2**-53 is two squares of 2**-27): the
    # pairwise tree gives (1 + 0) + (2**-53 + 2**-53) = 1 + 2**-52, where adding
    # the block sums one after the other gives 1.
    row = np.zeros((1, 128), np.float32)
    row[0, 0] = one
    row[0, 64:66] = small
    row[0, 96:98] = small
    assert rms_sum_sq_ref(_bits(row))[0] == 1.0 + 2.0 ** -52
    # a non-power-of-two block count pads with zero blocks: 3 blocks -> (b0 + b1) + (b2 + 0)
    row = np.zeros((1, 96), np.float32)
    row[0, 0] = one
    row[0, 32:34] = small
    row[0, 64:66] = small
    assert rms_sum_sq_ref(_bits(row))[0] == 1.0  # (1 + 2**-53) -> 1, (2**-53 + 0), 1 + 2**-53 -> 1


def test_prepare_with_rms_is_prepare_of_the_normalised_rows():
    rng = np.random.default_rng(8)
    x = _bits(rng.standard_normal((16, 512)) * 7)
    g = _bits(rng.uniform(0.5, 1.5, 512))
    xn, r = rms_normalize_ref(x, 1e-6)
    a = prepare_ref(x, g, 2, 4, rms_eps=1e-6)
    b = prepare_ref(xn, g, 2, 4)
    for k in ("mask", "bb_codes", "bb_scales", "res_codes", "res_scales"):
        assert np.array_equal(a[k], b[k])
    assert np.array_equal(a["rms_scale"], r)
    with pytest.raises(ValueError):
        rms_row_scale_ref(x, 0.0)
