"""Pins of the NVFP4 oracle (CPU only): E4M3 against torch's float8_e4m3fn
conversions, hand-worked blocks, invariants of the block coding, and the
two-path GEMM against the (separately pinned) MXFP4 oracle on inputs that both
formats carry exactly."""

import numpy as np
import pytest

from oracle import (decode_e2m1, e4m3_decode, e4m3_encode, linear_nvfp4_ref, linear_ref, nvfp4_dequantize,
                    nvfp4_quantize, pack_nibbles, prepare_nvfp4_ref, quantize_weight_nvfp4_ref,
                    tensor_scale_from_amax, unpack_mask, unpack_nibbles)
from synth import bf16_round, bf16_to_f32

torch = pytest.importorskip("torch")

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def torch_e4m3_bytes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_and_landmarks():
    b = np.arange(0x7F, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(e4m3_decode(b), want)
    assert e4m3_decode(np.array([0x7E]))[0] == 448.0          # largest finite
    assert e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9      # smallest subnormal
    assert e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6      # smallest normal
    assert e4m3_decode(np.array([0x38]))[0] == 1.0
    with pytest.raises(ValueError):
        e4m3_decode(np.array([0x7F]))  # NaN byte


def test_e4m3_encode_matches_torch_rne():
    vals = e4m3_decode(np.arange(0x7F)).astype(np.float32)
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(3)
    rnd = np.exp2(rng.uniform(-12, np.log2(448.0), 20000)).astype(np.float32)
    v = np.concatenate([vals, mids, up, dn, rnd, np.float32([0.0, 464.0, 2.0 ** -10, 2.0 ** -11])])
    assert np.array_equal(e4m3_encode(v), torch_e4m3_bytes(v))
    # the reading: saturation instead of NaN above 448
    big = np.float32([448.0001, 470.0, 1e6, 3e38, np.inf])
    assert np.all(e4m3_encode(big) == 0x7E)


def test_tensor_scale_from_amax():
    assert tensor_scale_from_amax(2688.0) == np.float32(1.0)
    assert tensor_scale_from_amax(0.0) == np.float32(1.0)
    assert tensor_scale_from_amax(6 * 448 * 2.0 ** -5) == np.float32(2.0 ** -5)


def block16(*head):
    x = np.zeros((1, 16), np.float32)
    x[0, :len(head)] = head
    return x


def test_hand_worked_blocks():
    # amax 7.5, s_t = 1: v = 7.5 / 6 = 1.25 = E4M3 0x3A (2^0 * (1 + 2/8)); d = 1.25;
    # 7.5/d = 6 -> code 7; -3/d = -2.4 -> 2 (code 4, sign) ; 0.1/d = 0.08 -> 0; 1.3/d = 1.04 -> 1 (code 2)
    c, s = nvfp4_quantize(block16(7.5, -3.0, 0.1, 1.3), 1.0)
    assert s[0, 0] == 0x3A
    assert list(c[0, :5]) == [7, 0xC, 0, 2, 0]
    # amax 6, s_t = 1: scale 1.0 (0x38); ties go to the even code: 5 -> 4 (code 6), 0.25 -> 0, 2.5 -> 2 (code 4),
    # -0.75 -> -1 (code 0xA, 1.0 has the even code 2 against 0.5's 1), 1.25 -> 1 (code 2)
    c, s = nvfp4_quantize(block16(6.0, 5.0, 0.25, 2.5, -0.75, 1.25), 1.0)
    assert s[0, 0] == 0x38
    assert list(c[0, :6]) == [7, 6, 0, 4, 0xA, 2]
    # the scale itself rounds to nearest even: amax 6.375 -> v = 1.0625, halfway between 1.0 (0x38) and
    # 1.125 (0x39) -> 0x38; then 6.375 / 1 saturates at 6
    c, s = nvfp4_quantize(block16(6.375), 1.0)
    assert s[0, 0] == 0x38 and c[0, 0] == 7
    # scale saturation: s_t = 2^-10, amax 6 -> v = 1024 > 448 -> 0x7E; d = 448 * 2^-10 = 0.4375; 6 / d = 13.7 -> 6
    c, s = nvfp4_quantize(block16(6.0, 0.4375), 2.0 ** -10)
    assert s[0, 0] == 0x7E and c[0, 0] == 7 and c[0, 1] == 2
    # subnormal scale: amax 18 * 2^-9 -> v = 3 * 2^-9 = E4M3 subnormal byte 3
    c, s = nvfp4_quantize(block16(18 * 2.0 ** -9, -3 * 2.0 ** -9), 1.0)
    assert s[0, 0] == 3 and c[0, 0] == 7 and c[0, 1] == 0xA
    # a block whose scale rounds to 0 (v = 2^-11 < 2^-10): every entry a signed zero
    c, s = nvfp4_quantize(block16(6 * 2.0 ** -11, -6 * 2.0 ** -11, -0.0), 1.0)
    assert s[0, 0] == 0 and list(c[0, :3]) == [0, 8, 8]
    # a non-power-of-two tensor scale: s_t = 0.3, amax 3.6 -> t6 = 1.8, v = 2 -> 0x40, d = fp32(2 * 0.3)
    c, s = nvfp4_quantize(block16(3.6, -0.9), 0.3)
    d = np.float32(np.float32(2.0) * np.float32(0.3))
    assert s[0, 0] == 0x40
    assert c[0, 0] == 7  # 3.6 / 0.6 = 6 (up to fp32 rounding, well inside the 4..6 interval)
    assert decode_e2m1(c[0, 1]) == -1.5 and abs(-0.9 / d + 1.5) < 1e-6


def test_block_invariants_random():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    for s_t in (1.0, 0.3, 2.0 ** -6, tensor_scale_from_amax(np.abs(x).max())):
        c, sb = nvfp4_quantize(x, s_t)
        amax = np.abs(x).reshape(64, -1, 16).max(-1)
        v = (amax / np.float32(np.float32(6) * np.float32(s_t))).astype(np.float32)
        # the scale byte is torch's float8_e4m3fn cast of v where v is in range
        ok = v <= 448
        assert np.array_equal(sb[ok], torch_e4m3_bytes(v[ok]))
        d = (e4m3_decode(sb).astype(np.float32) * np.float32(s_t)).astype(np.float32)
        q = (x / np.repeat(d, 16, axis=1)).astype(np.float64)
        vals = decode_e2m1(c)
        # no grid value is nearer to x / d than the chosen one (saturation aside)
        inside = np.abs(q) <= 6
        dist = np.abs(np.abs(q)[..., None] - E2M1[None, None, :]).min(-1)
        assert np.all(np.abs(np.abs(q) - np.abs(vals))[inside] == dist[inside])
        assert np.all(np.abs(vals[~inside]) == 6)
        assert np.array_equal(np.signbit(vals), np.signbit(x))
        # in a normal, unsaturated scale the block's largest entry codes as 6
        normal = (sb >= 0x08) & (v < 448)
        top = np.abs(x).reshape(64, -1, 16).argmax(-1)
        top_codes = np.take_along_axis(c.reshape(64, -1, 16), top[..., None], -1)[..., 0] & 7
        assert np.all(top_codes[normal] == 7)


def test_weight_quantizer_is_the_block_coding():
    rng = np.random.default_rng(9)
    w_bits = bf16_round((rng.standard_normal((8, 64)) * 0.02).astype(np.float32))
    w = bf16_to_f32(w_bits)
    s_w = tensor_scale_from_amax(np.abs(w).max())
    wc, ws = quantize_weight_nvfp4_ref(w_bits, s_w)
    c, s = nvfp4_quantize(w, s_w)
    assert np.array_equal(wc, pack_nibbles(c)) and np.array_equal(ws, s)
    err = np.abs(nvfp4_dequantize(c, s, s_w) - w)
    assert err.max() <= np.abs(w).max() / 6 * 1.0625  # at most one E2M1 step (2) times d / 2 in the top interval


def test_prepare_exact_case():
    """Kept entries that NVFP4 holds exactly (a block maximum of 6 * 2^j and every
    kept value on the E2M1 grid times 2^j, s_a = 1): the backbone is exact, so the
    residual is 0 at kept positions and x' at dropped ones."""
    rng = np.random.default_rng(11)
    T, K = 4, 64
    x = np.zeros((T, K), np.float32)
    for t in range(T):
        for g in range(K // 4):
            j = (t + g // 4) % 5 - 2
            kept = rng.choice([0.5, 1.0, 1.5, 2.0, 3.0, 4.0], 2) * 2.0 ** j
            small = rng.uniform(0, 0.25, 2) * 2.0 ** j  # strictly smaller: dropped under 2:4
            vals = np.concatenate([kept, small]) * rng.choice([-1, 1], 4)
            x[t, 4 * g:4 * g + 4] = vals[rng.permutation(4)]
        for b in range(K // 16):  # put the block maximum 6 * 2^j on a kept position
            blk = x[t, 16 * b:16 * b + 16]
            i = int(np.abs(blk).argmax())
            j = (t + (16 * b + i) // 16) % 5 - 2
            blk[i] = np.sign(blk[i]) * 6.0 * 2.0 ** j
    x_bits = bf16_round(x)  # kept values are exact in bf16; dropped ones stay below a quarter of theirs
    x = bf16_to_f32(x_bits)
    out = prepare_nvfp4_ref(x_bits, None, 2, 4, 1.0, keep_intermediates=True)
    keep = out["keep"]
    assert np.all(keep.reshape(T, -1, 4).sum(-1) == 2)
    assert np.array_equal(unpack_mask(out["mask"]), keep)
    assert np.all(out["r"][keep] == 0)
    assert np.array_equal(out["r"][~keep], x[~keep])
    assert np.all(unpack_nibbles(out["bb_codes"])[~keep] == 0)


def test_prepare_reconstruction_bound():
    """x' - deq(backbone) - deq(residual) is the residual's own coding error: at
    most half an E2M1 step of the residual's block (or the saturation excess)."""
    from synth.workloads import _streams, outlier_activation
    rx, rc, rt = _streams(5, 3)
    x_bits = bf16_round(outlier_activation(rx, rc, rt, 32, 512))
    s_a = tensor_scale_from_amax(np.abs(bf16_to_f32(x_bits)).max())
    for n, m in ((2, 4), (8, 16)):
        out = prepare_nvfp4_ref(x_bits, None, n, m, s_a, keep_intermediates=True)
        bb = nvfp4_dequantize(unpack_nibbles(out["bb_codes"]), out["bb_scales"], s_a)
        rs = nvfp4_dequantize(unpack_nibbles(out["res_codes"]), out["res_scales"], s_a)
        err = np.abs(out["xp"].astype(np.float64) - bb - rs)
        d_r = np.repeat(e4m3_decode(out["res_scales"]) * np.float64(s_a), 16, axis=1)
        # |x' - bb - rs| <= |x' - q - r| (the fp32 subtraction) + |q - bb| (q's one rounding) + |r - rs|,
        # and |r - rs| is at most half the widest E2M1 step (2) times d_r, saturation included
        xp, q, r = (out[k].astype(np.float64) for k in ("xp", "q", "r"))
        assert np.all(err <= d_r + np.abs(xp - q - r) + np.abs(q - bb))
        # the residual path removes most of the backbone-only error
        e_bb = np.linalg.norm(out["xp"] - bb)
        assert np.linalg.norm(err) < 0.2 * e_bb


def _pow2_nvfp4(rng, rows, K, lo, hi):
    """Random codes with scale bytes that are powers of two and equal within
    each 32-block: (codes [rows, K], nv bytes [rows, K/16], mx bytes [rows, K/32])."""
    c = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    j = rng.integers(lo, hi + 1, (rows, K // 32))
    nv = np.repeat(((j + 7) << 3).astype(np.uint8), 2, axis=1)
    return c, nv, (j + 127).astype(np.uint8)


def test_linear_matches_mxfp4_oracle_on_shared_values():
    rng = np.random.default_rng(13)
    T, O, K = 5, 7, 128
    bc, bnv, bmx = _pow2_nvfp4(rng, T, K, -6, 8)
    rcd, rnv, rmx = _pow2_nvfp4(rng, T, K, -6, 2)
    wc, wnv, wmx = _pow2_nvfp4(rng, O, K, -6, 0)
    y_nv, b_nv = linear_nvfp4_ref(pack_nibbles(bc), bnv, pack_nibbles(rcd), rnv, 1.0, pack_nibbles(wc), wnv, 1.0)
    y_mx, b_mx = linear_ref(pack_nibbles(bc), bmx, pack_nibbles(rcd), rmx, pack_nibbles(wc), wmx)
    assert np.array_equal(y_nv, y_mx) and np.array_equal(b_nv, b_mx)
    # tensor scales multiply through exactly (powers of two)
    y2, _ = linear_nvfp4_ref(pack_nibbles(bc), bnv, pack_nibbles(rcd), rnv, 0.25, pack_nibbles(wc), wnv, 8.0)
    assert np.array_equal(y2, 2.0 * y_mx)


def test_linear_block_mantissa_by_hand():
    """One row, one output, K = 32: two 16-blocks with scales 1.5 (0x3C) and
    0.875 (0x36), backbone codes 6 and -1 at the first entry of each block,
    residual zero, weight all 0.5 (code 1) with scale 1.0, s_a = 0.5, s_w = 2:
    Y = 0.5 * 2 * (6 * 1.5 * 0.5 + (-1) * 0.875 * 0.5) = 4.0625."""
    c = np.zeros((1, 32), np.uint8)
    c[0, 0], c[0, 16] = 7, 0xA
    sb = np.array([[0x3C, 0x36]], np.uint8)
    wc = np.ones((1, 32), np.uint8)
    ws = np.array([[0x38, 0x38]], np.uint8)
    zero = np.zeros((1, 16), np.uint8)
    y, b = linear_nvfp4_ref(pack_nibbles(c), sb, zero, sb, 0.5, pack_nibbles(wc), ws, 2.0)
    assert y[0, 0] == 4.0625 and b[0, 0] == 0.5 * 2 * (9 * 0.5 + 0.875 * 0.5)
