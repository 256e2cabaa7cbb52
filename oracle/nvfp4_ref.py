"""Oracle of SharQ on NVFP4, the second block-FP4 format (test infrastructure
only: the same rules as ``sharq_ref`` apply -- only tests, smoke() and the
bench's CPU baseline may call it, and it shares nothing with the HIP library).

What the pages fix: the SharQ page (Abstract) says the method generalises to
NVFP4 as well as MXFP4; the decomposition itself (N:M backbone, residual
against the quantised backbone, both paths in FP4 against one FP4 weight) is
the one of ``sharq_ref``. The pages never define NVFP4. The plain reading
used here is its public definition:

* elements are E2M1 (the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit),
  in blocks of 16 consecutive entries along K;
* each block has one FP8 E4M3 scale (OCP "E4M3FN": bias 7, 3 mantissa bits,
  largest finite 448, smallest subnormal 2^-9, bytes 0x7F/0xFF are NaN);
* each tensor has one fp32 scale s_t on top, so that an entry decodes to
  e2m1(code) * e4m3(block scale) * s_t.

Readings taken where the public description leaves steps open, all
arithmetic in fp32 with round-to-nearest-even unless stated:
* block scale: v = amax_block / fp32(6 * s_t) (a correctly rounded division),
  then the E4M3 value nearest to v, ties to the even code, saturated to 448
  (never NaN); amax is over the entries being coded (the kept ones for the
  backbone);
* element code: with d = fp32(e4m3(scale) * s_t), the E2M1 code nearest to
  fp32(x / d), ties to the even code, saturated at 6, sign kept on zero; a
  block whose d is 0 codes every entry as a signed zero;
* the activation has one tensor scale s_a shared by the backbone and the
  residual (two encodings of parts of one tensor; each keeps its own block
  scales); the weight has its own s_w. Both are inputs (static calibration,
  the usual practice for activations); ``tensor_scale_from_amax`` gives the
  common choice amax / (6 * 448);
* the residual is r = fp32(x' - fp32(e2m1 * e4m3 * s_a)) (the dequantised
  backbone rounded once to fp32, then one subtraction);
* the GEMM is Y = deq(A_s) deq(W)^T + deq(A_r) deq(W)^T, like the MXFP4 one.

Parity pins (tests/test_oracle_nvfp4.py): E4M3 decode and encode against
torch's float8_e4m3fn conversions, hand-worked blocks, the block-maximum and
error-bound invariants, exact decompositions, and the GEMM against the pinned
MXFP4 oracle on inputs where both formats carry the same values.
"""

from __future__ import annotations

import numpy as np

from .sharq_ref import (absorb_gamma, decode_e2m1, pack_mask, pack_nibbles, quantize_e2m1, select_nm,
                        unpack_nibbles)

__all__ = ["NV_BLOCK", "E4M3_MAX", "e4m3_decode", "e4m3_encode", "tensor_scale_from_amax", "nvfp4_quantize",
           "nvfp4_dequantize", "prepare_nvfp4_ref", "quantize_weight_nvfp4_ref", "linear_nvfp4_ref"]

NV_BLOCK = 16
E4M3_MAX = 448.0


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """E4M3 byte (sign clear, 0x00..0x7E) -> float64: exponent field e, mantissa
    m; e > 0: 2^(e-7) (1 + m/8); e == 0: m 2^-9."""
    b = np.asarray(b, dtype=np.int64)
    if np.any((b < 0) | (b > 0x7E)):
        raise ValueError("not a finite non-negative E4M3 byte")
    e, m = b >> 3, b & 7
    return np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m.astype(np.float64), -9))


_E4M3_CODES = np.arange(0x7F)
_E4M3_VALUES = e4m3_decode(_E4M3_CODES)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Non-negative float32 values -> the byte of the nearest E4M3 value, ties
    to the even code; everything above 448 (+inf included) gives 448 (0x7E)."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(np.isnan(v)) or np.any(v < 0):
        raise ValueError("e4m3_encode takes non-negative values")
    flat = np.minimum(v.reshape(-1), E4M3_MAX)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 16
    for s in range(0, flat.size, step):
        vv = flat[s:s + step]
        d = np.abs(vv[:, None] - _E4M3_VALUES[None, :])
        cand = d == d.min(axis=1, keepdims=True)
        even = cand & ((_E4M3_CODES[None, :] & 1) == 0)
        out[s:s + step] = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return out.reshape(v.shape)


def tensor_scale_from_amax(amax: float) -> np.float32:
    """The usual NVFP4 tensor scale amax / (6 * 448) in fp32 (1 for amax = 0)."""
    a = np.float32(amax)
    if not np.isfinite(a) or a < 0:
        raise ValueError("amax must be finite and non-negative")
    return np.float32(1.0) if a == 0 else np.float32(a / np.float32(6.0 * 448.0))


def nvfp4_quantize(vals: np.ndarray, s_t, keep: np.ndarray | None = None):
    """NVFP4 along the last axis: (codes uint8 [T, K], scale bytes uint8 [T, K/16]).

    Per 16-block: amax over the coded entries, v = amax / fp32(6 s_t), scale =
    e4m3_encode(v), d = fp32(e4m3(scale) s_t), code = quantize_e2m1(fp32(x / d))
    (all-signed-zero when d == 0); entries outside ``keep`` get code 0x0.
    """
    vals = np.asarray(vals, dtype=np.float32)
    s_t = np.float32(s_t)
    if not (np.isfinite(s_t) and s_t > 0):
        raise ValueError("tensor scale must be finite and positive")
    T, K = vals.shape
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    if keep is None:
        keep = np.ones(vals.shape, dtype=bool)
    nb = K // NV_BLOCK
    a = np.where(keep, np.abs(vals), np.float32(0)).reshape(T, nb, NV_BLOCK)
    amax = a.max(axis=-1)
    with np.errstate(over="ignore"):
        t6 = np.float32(np.float32(6.0) * s_t)
        v = (amax / t6).astype(np.float32)
    sb = e4m3_encode(v)
    d = (e4m3_decode(sb).astype(np.float32) * s_t).astype(np.float32)  # [T, nb]
    d_full = np.repeat(d, NV_BLOCK, axis=1)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = np.where(d_full > 0, vals / np.where(d_full > 0, d_full, np.float32(1)), np.float32(0))
    q = q.astype(np.float32)
    # beyond 6 every value codes as 6; an fp32 overflow of x / d (tiny d) is one
    codes = quantize_e2m1(np.clip(q.astype(np.float64), -7.0, 7.0))
    # d == 0: every entry a signed zero (its sign bit only)
    codes = np.where(d_full > 0, codes, (np.signbit(vals).astype(np.uint8) << 3))
    codes = np.where(keep, codes, np.uint8(0)).astype(np.uint8)
    return codes, sb


def nvfp4_dequantize(codes: np.ndarray, sb: np.ndarray, s_t) -> np.ndarray:
    """codes [T, K], scale bytes [T, K/16] -> float64 e2m1 * e4m3 * s_t (exact)."""
    scale = e4m3_decode(sb) * np.float64(np.float32(s_t))
    return decode_e2m1(codes) * np.repeat(scale, NV_BLOCK, axis=1)


def prepare_nvfp4_ref(x_bits: np.ndarray, gamma_bits: np.ndarray | None, n: int, m: int, s_a,
                      keep_intermediates: bool = False) -> dict:
    """The prepare operator with NVFP4 codes, on a [T, K] bf16 activation.

    Steps as ``prepare_ref``: x' = x * gamma, N:M mask on |x'|, backbone = kept
    entries in NVFP4, residual = fp32(x' - fp32(deq(backbone))), residual in
    NVFP4 over every entry with its own block scales; both with tensor scale
    s_a. Returns packed ``mask`` [T, K/8], ``bb_codes``/``res_codes`` [T, K/2]
    and ``bb_scales``/``res_scales`` [T, K/16] (E4M3 bytes).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, K = x_bits.shape
    if K % 32 or K % m:
        raise ValueError("K must be a multiple of 32 and of m")
    s_a = np.float32(s_a)
    xp = absorb_gamma(x_bits, gamma_bits)
    keep = select_nm(xp, n, m)
    bb_c, bb_s = nvfp4_quantize(xp, s_a, keep)
    # dequantised backbone: e2m1 * e4m3 is exact in fp32; one rounding for * s_a
    ev = (decode_e2m1(bb_c) * np.repeat(e4m3_decode(bb_s), NV_BLOCK, axis=1)).astype(np.float32)
    q = (ev * s_a).astype(np.float32)
    r = (xp - q).astype(np.float32)
    rs_c, rs_s = nvfp4_quantize(r, s_a, None)
    out = {"mask": pack_mask(keep), "bb_codes": pack_nibbles(bb_c), "bb_scales": bb_s,
           "res_codes": pack_nibbles(rs_c), "res_scales": rs_s}
    if keep_intermediates:
        out.update(xp=xp, keep=keep, q=q, r=r, bb_c=bb_c, rs_c=rs_c)
    return out


def quantize_weight_nvfp4_ref(w_bits: np.ndarray, s_w) -> tuple[np.ndarray, np.ndarray]:
    """NVFP4 of a bf16 weight [O, K] along K: (codes [O, K/2], E4M3 bytes [O, K/16])."""
    w32 = absorb_gamma(np.asarray(w_bits, dtype=np.uint16), None)
    c, s = nvfp4_quantize(w32, s_w, None)
    return pack_nibbles(c), s


def linear_nvfp4_ref(bb_codes, bb_scales, res_codes, res_scales, s_a, w_codes, w_scales, s_w):
    """Y = deq(A_s) deq(W)^T + deq(A_r) deq(W)^T in float64, with
    B = (|A_s| + |A_r|) |W|^T, the per-element bound the tolerance scales by."""
    a_s = nvfp4_dequantize(unpack_nibbles(bb_codes), bb_scales, s_a)
    a_r = nvfp4_dequantize(unpack_nibbles(res_codes), res_scales, s_a)
    w = nvfp4_dequantize(unpack_nibbles(w_codes), w_scales, s_w)
    y = a_s @ w.T + a_r @ w.T
    bound = (np.abs(a_s) + np.abs(a_r)) @ np.abs(w).T
    return y, bound
