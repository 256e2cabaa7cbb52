"""Plain, slow, obviously-correct CPU oracle of the SharQ linear hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code, tables or helpers with the HIP library, and it never reads a value the
HIP library produced, except where a chained stage is deliberately fed the GPU's
output of the previous stage (documented at the call site in the tests).

Sources (cited by page title and section):

* [SharQ] "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
  Inference" (Chinese translation of arXiv 2606.26587).
  - Abstract: per activation tensor, an input-adaptive N:M mask extracts an
    outlier-dominated sparse backbone that is quantised to FP4; a dense
    residual is defined relative to the *quantised* backbone; a sparse FP4 GEMM
    runs the backbone and a dense FP4 GEMM compensates both the masked-out
    activations and the sparse path's quantisation error; both paths share one
    FP4 weight; one fused prepare operator builds mask and residual and
    absorbs the layer norm.
  - Section 1 (Introduction): the residual therefore holds the values outside
    the mask plus the sparse path's FP4 quantisation error; the dense residual
    GEMM accumulates into the sparse output.
  - Section 2.3 (fine-grained numeric formats): MXFP4 is the OCP MX block-scaled
    format. The pages do not restate its rules; the plain reading used here is
    E2M1 elements {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit, 32-element
    blocks along K, one E8M0 power-of-two scale per block with exponent
    floor(log2(amax)) - 2 (E2M1's largest exponent is 2), round to nearest with
    ties to the even code, saturation at 6.
* [Challenge] "Huang Danian Chasi House list 137, problem 2: activation sparse
  quantisation based on N:M sparsity" (mhpn.cn), Module 1 (problem text): N:M on
  activations by top-k selection, 8:16 on down_proj; Module 6 step 1, formula 1:
  pruning rate = pruned elements / all elements.
* [8:16] "From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights
  with Variance Correction", key design: 8 of every 16 elements are kept.

Readings where the pages are silent:
  selection is on x' (after gamma); ties in |x'| go to the lower index; a group
  always keeps exactly N elements; scale blocks are 32 consecutive dense-K
  positions; an all-zero block gets exponent -127 (E8M0 byte 0x00); exponents
  clamp to [-127, 127]; a value that rounds to magnitude 0 keeps its sign;
  dropped positions carry code 0x0 (+0); the residual is kept in fp32; inputs
  must be finite.

Parity pins (tests/test_oracle_*.py): every public function below is pinned
against something other than itself -- brute-force enumeration, exhaustive
sweeps against numpy's own half-to-even rounding, closed forms and exact
invariants. ``silu_mul_ref`` is pinned against a 50-digit mpmath evaluation
of silu(g) * u rounded to bf16 by an independent midpoint search.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "E2M1_GRID",
    "bf16_bits_to_f32",
    "f64_to_bf16_bits_rne",
    "f32_to_bf16_bits_rne",
    "rms_sum_sq_ref",
    "rms_row_scale_ref",
    "rms_normalize_ref",
    "absorb_gamma",
    "select_nm",
    "floor_log2_f32",
    "block_scale_exponent",
    "quantize_e2m1",
    "decode_e2m1",
    "mxfp4_quantize",
    "mxfp4_dequantize",
    "pack_nibbles",
    "unpack_nibbles",
    "pack_mask",
    "unpack_mask",
    "prepare_ref",
    "quantize_weight_ref",
    "linear_ref",
    "linear_grouped_ref",
    "silu_mul_ref",
    "moe_combine_ref",
]

# E2M1 magnitudes indexed by the 3-bit code (bit 3 of a code is the sign).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
BLOCK = 32  # MX block length along K
E_MIN, E_MAX = -127, 127  # E8M0 exponent range used (byte 0xFF is never emitted)


def _require_finite(a: np.ndarray, what: str) -> None:
    if not np.all(np.isfinite(a)):
        raise ValueError(f"{what}: non-finite values are outside the method's domain")


# ---------------------------------------------------------------------------
# O1: input and gamma absorption  ([SharQ] Abstract: the fused prepare operator
# absorbs the layer norm; read as the per-channel RMSNorm gamma multiply)
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32. Exact: bf16 is the top half of fp32."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_to_bf16_bits_rne(h: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16, ties to the even significand.

    Written from the bf16 grid: in the binade of h (exponent e = floor(log2|h|))
    bf16 values are spaced 2**(e - 7), and below 2**-126 (the subnormal range)
    uniformly 2**-133; h / spacing is rounded half-to-even by numpy's ``rint``
    in one step from the float64 value and scaled back exactly. Finite inputs
    whose rounding stays finite in bf16 only.
    """
    h = np.asarray(h, dtype=np.float64)
    _require_finite(h, "f64_to_bf16_bits_rne")
    a = np.abs(h)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))  # a = f * 2**ex, f in [0.5, 1): e = ex - 1
    step_exp = np.maximum(ex - 1 - 7, -133)
    r = np.ldexp(np.rint(np.ldexp(h, -step_exp)), step_exp)  # exact in float64
    r32 = r.astype(np.float32)  # exact: r lies on the bf16 grid
    _require_finite(r32, "bf16 rounding")
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16_bits_rne(v32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16, ties to the even significand
    (float32 -> float64 is exact, then the bf16 grid rounding above)."""
    return f64_to_bf16_bits_rne(np.asarray(v32, dtype=np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# O0: full RMSNorm absorption (the norm step right before the path: [SharQ]
# Abstract, the fused prepare absorbs the layer norm). Reading: the model's
# RMSNorm, x_n = bf16(x * r) with r = 1 / sqrt(mean_k x_k**2 + eps) per row,
# then x' = x_n * gamma; the row's sum of squares is accumulated in float64 in
# a fixed order so that every implementation that follows the order gets the
# same bits.
# ---------------------------------------------------------------------------

def rms_sum_sq_ref(x_bits: np.ndarray) -> np.ndarray:
    """S = sum_k x_k**2 per row in float64, in this fixed order.

    Each square of a bf16 value is exact in float64. The 32 squares of each MX
    block are added in index order, one after the other, starting from 0; the
    block sums are then combined by a pairwise tree over blocks in index order
    (adjacent pairs (2i, 2i + 1), level by level), padded with zero blocks to a
    power of two.
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    _require_finite(x, "x")
    T, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    nb = K // BLOCK
    sq = (x * x).reshape(T, nb, BLOCK)
    blk = np.zeros((T, nb))
    for k in range(BLOCK):
        blk = blk + sq[:, :, k]
    npad = 1
    while npad < nb:
        npad *= 2
    tree = np.zeros((T, npad))
    tree[:, :nb] = blk
    while tree.shape[1] > 1:
        tree = tree[:, 0::2] + tree[:, 1::2]
    return tree[:, 0]


def rms_row_scale_ref(x_bits: np.ndarray, eps: float) -> np.ndarray:
    """Per-row RMSNorm scale r = fp32(1 / sqrt(S / K + eps)), eps > 0, with S
    from ``rms_sum_sq_ref``. The mean, the addition of eps (taken exactly from
    its float32 value), sqrt and the reciprocal are float64 operations, each
    correctly rounded; r is then rounded to float32."""
    eps = float(np.float32(eps))
    if not (eps > 0 and np.isfinite(eps)):
        raise ValueError("eps must be finite and > 0")
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    v = rms_sum_sq_ref(x_bits) / x_bits.shape[1] + eps
    return (1.0 / np.sqrt(v)).astype(np.float32)


def rms_normalize_ref(x_bits: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """x_n = bf16_rne(fp32(x) * r) per row: returns (x_n bf16 bits [T, K], r [T])."""
    r = rms_row_scale_ref(x_bits, eps)
    x32 = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    with np.errstate(under="ignore"):
        xr = (x32 * r[:, None]).astype(np.float32)
    return f32_to_bf16_bits_rne(xr), r


def absorb_gamma(x_bits: np.ndarray, gamma_bits: np.ndarray | None) -> np.ndarray:
    """x' = f32(x) * f32(gamma) in float32 (round to nearest even).

    The product of two bf16 values has at most 16 significant bits, so it is
    exact in float32 unless it falls in the float32 subnormal range, where IEEE
    gradual underflow rounds it.
    """
    x32 = bf16_bits_to_f32(x_bits)
    _require_finite(x32, "x")
    if gamma_bits is None:
        return x32
    g32 = bf16_bits_to_f32(gamma_bits)
    _require_finite(g32, "gamma")
    if g32.shape != (x32.shape[-1],):
        raise ValueError("gamma must have K entries")
    with np.errstate(under="ignore", over="ignore"):
        xp = (x32 * g32[None, :]).astype(np.float32)
    _require_finite(xp, "x * gamma")
    return xp


# ---------------------------------------------------------------------------
# O2: online N:M selection  ([SharQ] Abstract and Section 1: an input-adaptive
# N:M mask computed from the current activation; [Challenge] Module 1: top-k
# selection inside each group of M; [8:16] key design: 8 kept of each 16)
# ---------------------------------------------------------------------------

def select_nm(xp: np.ndarray, n: int, m: int) -> np.ndarray:
    """Boolean keep-mask: in each group of m consecutive K positions keep the n
    entries with the largest |x'|; equal magnitudes (including +0/-0 and values
    of opposite sign) go to the lower index. Exactly n kept per group."""
    xp = np.asarray(xp, dtype=np.float32)
    T, K = xp.shape
    if not (1 <= n <= m) or K % m:
        raise ValueError("need 1 <= n <= m and K % m == 0")
    a = np.abs(xp).reshape(T, K // m, m)
    # A stable sort on the negated magnitude lists larger |x'| first and keeps
    # equal magnitudes in ascending index order.
    order = np.argsort(-a, axis=-1, kind="stable")
    keep = np.zeros(a.shape, dtype=bool)
    np.put_along_axis(keep, order[..., :n], True, axis=-1)
    return keep.reshape(T, K)


# ---------------------------------------------------------------------------
# O3: E8M0 block scale  ([SharQ] Section 2.3, MX block scaling; [SharQ]
# Section 1: a block's scale is chosen from the block's largest value)
# ---------------------------------------------------------------------------

def floor_log2_f32(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite float32 a > 0, from the bit pattern (no log2f).

    Normal numbers: the unbiased exponent field. Subnormals: the position of the
    leading set mantissa bit, minus 149 (the subnormal LSB is 2**-149)."""
    a = np.asarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    expf = (bits >> 23) & 0xFF
    mant = bits & 0x7FFFFF
    # bit length of the mantissa, counted without floating point
    blen = np.zeros_like(mant)
    for j in range(23):
        blen += (mant >= (1 << j)).astype(np.int64)
    return np.where(expf > 0, expf - 127, blen - 1 - 149)


def block_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Block exponent e = clamp(floor(log2(amax)) - 2, -127, 127); amax == 0 -> -127."""
    amax = np.asarray(amax, dtype=np.float32)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1.0))
    e = floor_log2_f32(safe) - 2
    e = np.clip(e, E_MIN, E_MAX)
    return np.where(pos, e, E_MIN).astype(np.int64)


# ---------------------------------------------------------------------------
# O4: E2M1 element coding  ([SharQ] Section 2.3; plain reading of MXFP4)
# ---------------------------------------------------------------------------

def quantize_e2m1(v: np.ndarray) -> np.ndarray:
    """Code of the E2M1 value nearest to v (float64, finite).

    Magnitude: the nearest entry of E2M1_GRID; at an exact midpoint the even
    code wins; anything beyond 6 lands on 6 because 6 is the nearest grid entry.
    Sign: bit 3 copies v's sign bit, including for -0 and values that round to 0.
    """
    v = np.asarray(v, dtype=np.float64)
    _require_finite(v, "quantize_e2m1")
    # Beyond 6 the nearest grid point is 6 whatever the magnitude; capping at 7
    # keeps the distance arithmetic below exact in float64 for huge inputs.
    mag = np.minimum(np.abs(v), 7.0).reshape(-1)
    codes = np.empty(mag.shape, dtype=np.uint8)
    step = 1 << 20
    idx = np.arange(8)
    for s in range(0, mag.size, step):
        mm = mag[s:s + step]
        d = np.abs(mm[:, None] - E2M1_GRID[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among equally near grid points prefer an even code
        pref = cand & ((idx[None, :] % 2) == 0)
        pick = np.where(pref.any(axis=1), pref.argmax(axis=1), cand.argmax(axis=1))
        codes[s:s + step] = pick
    codes = codes.reshape(v.shape)
    codes |= (np.signbit(v).astype(np.uint8) << 3)
    return codes


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """E2M1 code -> float64 value."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[codes & 7]
    return np.where(codes & 8, -mag, mag)


def mxfp4_quantize(vals: np.ndarray, keep: np.ndarray | None = None):
    """MXFP4 along the last axis: returns (codes uint8 [T,K], exponents int64 [T,K/32]).

    For each 32-block: amax over the kept entries, e from ``block_scale_exponent``,
    code = quantize_e2m1(x * 2**-e) for kept entries and 0x0 for dropped ones.
    ``vals`` is float32; x * 2**-e is formed in float64 where it is exact.
    """
    vals = np.asarray(vals, dtype=np.float32)
    T, K = vals.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    if keep is None:
        keep = np.ones(vals.shape, dtype=bool)
    a = np.where(keep, np.abs(vals), np.float32(0)).reshape(T, K // BLOCK, BLOCK)
    e = block_scale_exponent(a.max(axis=-1))  # [T, K/32]
    scale = np.ldexp(1.0, -np.repeat(e, BLOCK, axis=1))  # float64 2**-e
    v = vals.astype(np.float64) * scale
    codes = quantize_e2m1(v)
    codes = np.where(keep, codes, np.uint8(0)).astype(np.uint8)
    return codes, e


def mxfp4_dequantize(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """codes [T,K] with exponents [T,K/32] -> float64 values val(code) * 2**e."""
    return decode_e2m1(codes) * np.ldexp(1.0, np.repeat(np.asarray(e, np.int64), BLOCK, axis=1))


# ---------------------------------------------------------------------------
# O7: packing (plain reading: low nibble holds the even K index; E8M0 byte is
# e + 127; mask bit (k & 7) of byte (k >> 3))
# ---------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def pack_mask(keep: np.ndarray) -> np.ndarray:
    keep = np.asarray(keep, dtype=bool)
    T, K = keep.shape
    bits = keep.reshape(T, K // 8, 8).astype(np.uint8)
    weights = (1 << np.arange(8)).astype(np.uint8)
    return (bits * weights).sum(axis=-1).astype(np.uint8)


def unpack_mask(mask_bytes: np.ndarray) -> np.ndarray:
    mb = np.asarray(mask_bytes, dtype=np.uint8)
    bits = (mb[:, :, None] >> np.arange(8, dtype=np.uint8)[None, None, :]) & 1
    return bits.reshape(mb.shape[0], mb.shape[1] * 8).astype(bool)


# ---------------------------------------------------------------------------
# The prepare operator, steps O1-O7 in the order [SharQ] Abstract and Section 1
# describe: mask -> quantised backbone -> residual against the quantised
# backbone -> residual quantised with its own scales.
# ---------------------------------------------------------------------------

def prepare_ref(x_bits: np.ndarray, gamma_bits: np.ndarray | None, n: int, m: int,
                keep_intermediates: bool = False, rms_eps: float | None = None) -> dict:
    """Oracle of the fused prepare operator on a [T, K] bf16 activation.

    Returns packed outputs ``mask`` [T,K/8], ``bb_codes`` [T,K/2],
    ``bb_scales`` [T,K/32], ``res_codes`` [T,K/2], ``res_scales`` [T,K/32]
    (all uint8). With ``rms_eps`` the full RMSNorm is absorbed first (O0:
    x is replaced by bf16(x * r), r returned as ``rms_scale`` float32 [T]).
    With ``keep_intermediates`` it also returns x', the boolean mask, the
    dequantised backbone q, the residual r and the unpacked codes.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, K = x_bits.shape
    if K % BLOCK or K % m:
        raise ValueError("K must be a multiple of 32 and of m")
    # O0
    rms = None
    if rms_eps is not None:
        x_bits, rms = rms_normalize_ref(x_bits, rms_eps)
    # O1
    xp = absorb_gamma(x_bits, gamma_bits)
    # O2
    keep = select_nm(xp, n, m)
    # O3 + O4: backbone = kept entries, quantised with block scales
    bb_c, bb_e = mxfp4_quantize(xp, keep)
    # dequantised backbone in float32 (exact: 2-bit significand times 2**e, e >= -127)
    q = mxfp4_dequantize(bb_c, bb_e).astype(np.float32)
    # O5: residual against the quantised backbone, fp32 round-to-nearest-even
    r = (xp - q).astype(np.float32)
    # O6: residual quantised over every position of the block, with its own scales
    rs_c, rs_e = mxfp4_quantize(r, None)
    out = {
        "mask": pack_mask(keep),
        "bb_codes": pack_nibbles(bb_c),
        "bb_scales": (bb_e + 127).astype(np.uint8),
        "res_codes": pack_nibbles(rs_c),
        "res_scales": (rs_e + 127).astype(np.uint8),
    }
    if rms is not None:
        out["rms_scale"] = rms
    if keep_intermediates:
        out.update(xp=xp, keep=keep, q=q, r=r, bb_c=bb_c, bb_e=bb_e, rs_c=rs_c, rs_e=rs_e)
    return out


def quantize_weight_ref(w_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Plain MXFP4 of a bf16 weight [O, K] along K: (codes [O,K/2], scale bytes [O,K/32])."""
    w32 = absorb_gamma(np.asarray(w_bits, dtype=np.uint16), None)
    c, e = mxfp4_quantize(w32, None)
    return pack_nibbles(c), (e + 127).astype(np.uint8)


# ---------------------------------------------------------------------------
# O8: the two-path GEMM  ([SharQ] Abstract: sparse FP4 GEMM on the backbone plus
# dense FP4 GEMM on the residual, one shared FP4 weight; Section 1: the residual
# path accumulates into the sparse output)
# ---------------------------------------------------------------------------

def _deq_packed(codes_packed, scale_bytes) -> np.ndarray:
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return mxfp4_dequantize(unpack_nibbles(codes_packed), e)


def linear_ref(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales):
    """Y = deq(backbone) @ deq(W)^T + deq(residual) @ deq(W)^T in float64.

    Returns (Y, B) where B = (|a_s| + |a_r|) @ |w|^T bounds the per-element
    sum of |a_k w_k| that the tolerance is scaled by.
    """
    a_s = _deq_packed(bb_codes, bb_scales)
    a_r = _deq_packed(res_codes, res_scales)
    w = _deq_packed(w_codes, w_scales)
    y = a_s @ w.T + a_r @ w.T
    bound = (np.abs(a_s) + np.abs(a_r)) @ np.abs(w).T
    return y, bound


def linear_grouped_ref(bb_codes, bb_scales, res_codes, res_scales, a_rows, seg_offsets,
                       w_codes, w_scales):
    """Grouped two-path GEMM: row p of the output uses source row a_rows[p] (or p
    when a_rows is None) and the weight of the expert whose segment holds p.

    w_codes [E, O, K/2], w_scales [E, O, K/32]; seg_offsets [E+1]. Returns (Y, B)
    with Y [P, O] in sorted-pair order."""
    seg = np.asarray(seg_offsets, dtype=np.int64)
    E = seg.size - 1
    P = int(seg[-1])
    rows = np.arange(P) if a_rows is None else np.asarray(a_rows, dtype=np.int64)
    O = np.asarray(w_codes).shape[1]
    y = np.zeros((P, O))
    bound = np.zeros((P, O))
    bbc, bbs = np.asarray(bb_codes), np.asarray(bb_scales)
    rsc, rss = np.asarray(res_codes), np.asarray(res_scales)
    for e in range(E):
        lo, hi = int(seg[e]), int(seg[e + 1])
        if hi <= lo:
            continue
        r = rows[lo:hi]
        ye, be = linear_ref(bbc[r], bbs[r], rsc[r], rss[r], w_codes[e], w_scales[e])
        y[lo:hi] = ye
        bound[lo:hi] = be
    return y, bound


# ---------------------------------------------------------------------------
# Glue between the gate|up and down projections (not the method itself)
# ---------------------------------------------------------------------------

def silu_mul_ref(gu: np.ndarray, inter: int) -> np.ndarray:
    """h = bf16_rne(silu(g) * u) with g = gu[:, :I], u = gu[:, I:2I], in float64."""
    gu = np.asarray(gu, dtype=np.float64)
    _require_finite(gu, "gu")
    g = gu[:, :inter]
    u = gu[:, inter:2 * inter]
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return f64_to_bf16_bits_rne(h)


def moe_combine_ref(y: np.ndarray, pair_index: np.ndarray, weights: np.ndarray):
    """Weighted combine of a mixture-of-experts layer (glue around the grouped
    two-path GEMM; the SharQ page, Abstract, names MoE models as targets):
    out[t] = sum over slots j of weights[t, j] * y[pair_index[t, j]], skipping
    slots with pair_index -1, in float64. Returns (out [T, H] float64, bound
    [T, H] = sum_j |weights[t, j] * y[pair_index[t, j]]|)."""
    y = np.asarray(y, dtype=np.float64)
    idx = np.asarray(pair_index)
    w = np.asarray(weights, dtype=np.float64)
    _require_finite(y, "y")
    T, k = idx.shape
    out = np.zeros((T, y.shape[1]))
    bound = np.zeros((T, y.shape[1]))
    for j in range(k):
        ok = idx[:, j] >= 0
        term = w[ok, j][:, None] * y[idx[ok, j]]
        out[ok] += term
        bound[ok] += np.abs(term)
    return out, bound
