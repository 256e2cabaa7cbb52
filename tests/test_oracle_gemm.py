"""Pins for the oracle's two-path GEMM (CPU only): exact rational triple loops on
tiny shapes, the single-GEMM (K-concatenated) form, and the grouped variant
against per-row evaluation."""

from fractions import Fraction

import numpy as np

from oracle import (decode_e2m1, linear_grouped_ref, linear_ref, prepare_ref,
                    quantize_weight_ref, unpack_nibbles, silu_mul_ref, f64_to_bf16_bits_rne)
from synth import bf16_round, bf16_to_f32, moe_routing


def _exact_value(code, scale_byte):
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
           Fraction(3), Fraction(4), Fraction(6)][code & 7]
    v = -mag if code & 8 else mag
    return v * Fraction(2) ** (int(scale_byte) - 127)


def _exact_matrix(codes_p, scales):
    c = unpack_nibbles(codes_p)
    return [[_exact_value(int(c[i, k]), scales[i, k // 32]) for k in range(c.shape[1])]
            for i in range(c.shape[0])]


def _setup(T, O, K, seed):
    rng = np.random.default_rng(seed)
    x = bf16_round((rng.standard_normal((T, K)) * rng.lognormal(0, 2, (T, 1))).astype(np.float32))
    w = bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32))
    p = prepare_ref(x, None, 2, 4)
    wc, ws = quantize_weight_ref(w)
    return p, wc, ws


def test_linear_against_exact_rational_loop():
    T, O, K = 3, 4, 64
    p, wc, ws = _setup(T, O, K, 0)
    y, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    A_s = _exact_matrix(p["bb_codes"], p["bb_scales"])
    A_r = _exact_matrix(p["res_codes"], p["res_scales"])
    W = _exact_matrix(wc, ws)
    for t in range(T):
        for o in range(O):
            exact = sum(A_s[t][k] * W[o][k] for k in range(K)) + sum(A_r[t][k] * W[o][k] for k in range(K))
            absum = sum(abs(A_s[t][k] * W[o][k]) + abs(A_r[t][k] * W[o][k]) for k in range(K))
            assert abs(Fraction(y[t, o]) - exact) <= Fraction(1, 10 ** 12) * absum
            assert abs(Fraction(bound[t, o]) - absum) <= Fraction(1, 10 ** 12) * absum


def test_two_paths_equal_one_concatenated_gemm_and_residual_zero_case():
    T, O, K = 5, 6, 128
    p, wc, ws = _setup(T, O, K, 1)
    y, _ = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    # K-concatenated single GEMM: [a_s | a_r] @ [w | w]^T
    def deq(cp, s):
        c = unpack_nibbles(cp)
        return decode_e2m1(c) * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    a = np.concatenate([deq(p["bb_codes"], p["bb_scales"]), deq(p["res_codes"], p["res_scales"])], axis=1)
    w = deq(wc, ws)
    y2 = a @ np.concatenate([w, w], axis=1).T
    assert np.allclose(y, y2, rtol=1e-13, atol=0)
    # residual forced to zero: a plain MXFP4 GEMM of the backbone
    zc = np.zeros_like(p["res_codes"])
    y3, _ = linear_ref(p["bb_codes"], p["bb_scales"], zc, p["res_scales"], wc, ws)
    assert np.allclose(y3, deq(p["bb_codes"], p["bb_scales"]) @ w.T, rtol=1e-13, atol=0)


def test_grouped_matches_per_row_linear():
    rng = np.random.default_rng(3)
    tokens, E, K, O = 40, 5, 64, 8
    x = bf16_round(rng.standard_normal((tokens, K)).astype(np.float32))
    p = prepare_ref(x, None, 2, 4)
    a_rows, seg, e_of_pair, _ = moe_routing(rng, tokens, E, 2)
    seg = seg.copy()
    wq = [quantize_weight_ref(bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32)))
          for _ in range(E)]
    wc = np.stack([c for c, _ in wq])
    ws = np.stack([s for _, s in wq])
    y, b = linear_grouped_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"],
                              a_rows, seg, wc, ws)
    for pidx in range(len(a_rows)):
        t, e = a_rows[pidx], e_of_pair[pidx]
        yy, bb = linear_ref(p["bb_codes"][t:t + 1], p["bb_scales"][t:t + 1], p["res_codes"][t:t + 1],
                            p["res_scales"][t:t + 1], wc[e], ws[e])
        assert np.array_equal(y[pidx], yy[0]) and np.array_equal(b[pidx], bb[0])
    # empty experts are allowed
    seg2 = np.array([0, 0, len(a_rows), len(a_rows), len(a_rows), len(a_rows)], np.int32)
    y2, _ = linear_grouped_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"],
                               a_rows, seg2, wc, ws)
    yy, _ = linear_ref(p["bb_codes"][a_rows], p["bb_scales"][a_rows], p["res_codes"][a_rows],
                       p["res_scales"][a_rows], wc[1], ws[1])
    assert np.array_equal(y2, yy)


def test_silu_mul_closed_forms_and_rounding():
    I = 6
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5])
    u = np.array([3.0, 1.0, 1.0, 2.0, 1.0, -1.0])
    h = bf16_to_f32(silu_mul_ref(np.concatenate([g, u])[None, :], I)[0]).astype(np.float64)
    want = g / (1 + np.exp(-g)) * u
    assert h[0] == 0.0
    assert abs(h[3] - 60.0) <= 60.0 * 2 ** -8
    # silu(-x) = silu(x) - x
    assert abs(h[2] - (h[1] - 1.0)) <= 2 ** -7
    # every result is the nearest bf16 to the float64 value (brute-force neighbour search)
    for val, hv in zip(want, h):
        if val == 0:
            continue
        b = int(f64_to_bf16_bits_rne(np.array([val]))[0])
        neighbours = bf16_to_f32(np.array([b - 1, b, b + 1], np.uint16)).astype(np.float64)
        d = np.abs(neighbours - val)
        assert d[1] <= d.min()
        assert hv == neighbours[1]


def test_bf16_rounding_ties_to_even():
    # 1 + 2**-8 is exactly halfway between bf16 1.0 and 1 + 2**-7: goes to 1.0 (even)
    assert f64_to_bf16_bits_rne(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3 * 2**-8 is halfway between 1 + 2**-7 and 1 + 2**-6: goes to 1 + 2**-6 (even)
    assert f64_to_bf16_bits_rne(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82
    assert f64_to_bf16_bits_rne(np.array([-0.0]))[0] == 0x8000


def _mp_bf16_bits(v, zero_sign=False):
    """The bf16 nearest to the mpmath value v (ties to the even significand),
    found by bracketing v between adjacent bf16 values of its binade and
    comparing against their midpoint in mpmath arithmetic. mpmath has no
    signed zero: an exact zero takes the sign `zero_sign` (IEEE's sign rule
    for the operation that produced it)."""
    import mpmath
    if v == 0:
        return 0x8000 if zero_sign else 0
    neg = v < 0
    a = -v if neg else v
    m, ex = mpmath.frexp(a)            # a = m * 2**ex, m in [0.5, 1)
    step = max(int(ex) - 1 - 7, -133)  # bf16 spacing in this binade (subnormal grid below 2**-126)
    q = a / mpmath.mpf(2) ** step
    lo = int(mpmath.floor(q))
    mid = mpmath.mpf(lo) + mpmath.mpf(1) / 2
    n = lo + 1 if q > mid else lo if q < mid else (lo if lo % 2 == 0 else lo + 1)
    r = np.float32(float(mpmath.mpf(n) * mpmath.mpf(2) ** step))  # exact: n has at most 9 bits
    bits = int(r.view(np.uint32)) >> 16
    return bits | (0x8000 if neg else 0)


def test_silu_mul_against_mpmath():
    """silu_mul_ref on float32 (g, u) pairs equals silu(g) * u evaluated with 50
    significant digits and rounded to bf16 by a midpoint search, including
    |g| >= 80 (results in bf16's subnormal range and exact zeros) and ties."""
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(7)
    g = np.concatenate([rng.standard_normal(2000) * 3, rng.uniform(-120, -80, 300), rng.uniform(80, 120, 300),
                        rng.uniform(-20, 20, 400), [0.0, -0.0, 1.0, -1.0, 88.5, -88.5, -103.0]]).astype(np.float32)
    u = np.concatenate([rng.standard_normal(2000) * 2, rng.uniform(-1e3, 1e3, 300), rng.standard_normal(300),
                        rng.standard_normal(400) * 1e-3, [1.0, 2.0, 3.0, -1.0, 1.0, 1e30, 1e30]]).astype(np.float32)
    I = len(g)
    got = silu_mul_ref(np.concatenate([g, u])[None, :], I)[0]
    want = []
    for gi, ui in zip(g.astype(np.float64), u.astype(np.float64)):
        G, U = mpmath.mpf(gi), mpmath.mpf(ui)
        # silu(+-0) = +-0 / 2, and a product of zeros carries the xor of the signs
        want.append(_mp_bf16_bits(G / (1 + mpmath.exp(-G)) * U, bool(np.signbit(gi) ^ np.signbit(ui))))
    want = np.array(want, dtype=np.uint16)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first g={g[bad[0]]} u={u[bad[0]]}: {got[bad[0]]:#06x} " \
                          f"vs {want[bad[0]]:#06x}"
    # the sample reaches the subnormal range and the signed zeros
    assert np.any((want & 0x7F80) == 0) and np.any(want == 0x8000)


def test_bf16_rounding_subnormal_grid():
    """Below 2**-126 bf16 values are spaced 2**-133: the rounding stays on that grid."""
    tiny = 2.0 ** -133
    assert f64_to_bf16_bits_rne(np.array([tiny]))[0] == 0x0001
    assert f64_to_bf16_bits_rne(np.array([0.5 * tiny]))[0] == 0x0000          # tie -> even (zero)
    assert f64_to_bf16_bits_rne(np.array([1.5 * tiny]))[0] == 0x0002          # tie -> even
    assert f64_to_bf16_bits_rne(np.array([-2.4 * tiny]))[0] == 0x8002
    assert f64_to_bf16_bits_rne(np.array([127.5 * tiny]))[0] == 0x0080        # tie -> 128 = 2**-126 (normal)
