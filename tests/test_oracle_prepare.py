"""Pins for the oracle's prepare operator (CPU only): a hand-worked block,
exact invariants of the decomposition, and special cases that reduce to plain
MXFP4 quantisation."""

import numpy as np
import pytest

from oracle import (absorb_gamma, mxfp4_dequantize, mxfp4_quantize, pack_nibbles,
                    prepare_ref, unpack_mask, unpack_nibbles)
from synth import adversarial_rows, bf16_round, bf16_to_f32, workload_down_silu, workload_linear


def test_hand_worked_2of4_block():
    # One 32-element row, worked by hand (derivation in the comments):
    #  g0 [1, -3, .5, 2]  keeps -3, 2           nibble 0b1010
    #  g1 [.25]*4         ties keep k=0,1       0b0011
    #  g2 [-6, 0, 0, 0]   keeps -6 and the first zero  0b0011
    #  g3 [.75,-.75,1.25,0] keeps 1.25 and the first .75  0b0101
    #  g4..g7 zeros       0b0011
    # backbone amax 6 -> floor(log2 6) - 2 = 0 -> byte 127, scale 1:
    #  -3 -> 0xD, 2 -> 0x4, .25 -> 0 (tie to even), -6 -> 0xF, .75 -> 1.0 (0x2), 1.25 -> 1.0 (0x2)
    # residual r = x - q: g0 [1,0,.5,0], g1 [.25]*4, g2 0, g3 [-.25,-.75,.25,0]
    # residual amax 1 -> e = -2 -> byte 125, v = 4r:
    #  g0 [4,0,2,0] -> 6,0,4,0; g1 [1]*4 -> 2; g3 [-1,-3,1,0] -> 0xA,0xD,0x2,0
    x = np.zeros((1, 32), np.float32)
    x[0, :16] = [1, -3, .5, 2, .25, .25, .25, .25, -6, 0, 0, 0, .75, -.75, 1.25, 0]
    out = prepare_ref(bf16_round(x), None, 2, 4)
    assert out["mask"].tolist() == [[0x3A, 0x53, 0x33, 0x33]]
    assert out["bb_scales"].tolist() == [[127]]
    assert out["bb_codes"].tolist() == [[0xD0, 0x40, 0, 0, 0x0F, 0, 0x02, 0x02] + [0] * 8]
    assert out["res_scales"].tolist() == [[125]]
    assert out["res_codes"].tolist() == [[0x06, 0x04, 0x22, 0x22, 0, 0, 0xDA, 0x02] + [0] * 8]


CASES = [
    ("2of4", 2, 4),
    ("8of16", 8, 16),
]


def _inputs(K, seed):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((20, K)) * rng.lognormal(0, 1, (20, 1))).astype(np.float32)
    base[:, rng.choice(K, 3, replace=False)] *= 50
    return bf16_round(np.concatenate([base, adversarial_rows(K, seed)]))


@pytest.mark.parametrize("name,n,m", CASES)
@pytest.mark.parametrize("with_gamma", [False, True])
def test_decomposition_invariants(name, n, m, with_gamma):
    K = 256
    xb = _inputs(K, 4)
    rng = np.random.default_rng(8)
    gamma = bf16_round(rng.uniform(0.5, 1.5, K).astype(np.float32)) if with_gamma else None
    out = prepare_ref(xb, gamma, n, m, keep_intermediates=True)
    xp, keep, q, r = out["xp"], out["keep"], out["q"], out["r"]
    # exactly n kept per group; mask packing round-trips
    assert np.all(keep.reshape(len(xb), -1, m).sum(-1) == n)
    assert np.array_equal(unpack_mask(out["mask"]), keep)
    # reconstruction is exact in float32 before the residual is quantised
    assert np.array_equal((q + r).astype(np.float32), xp)
    assert np.array_equal(q.astype(np.float64) + r.astype(np.float64), xp.astype(np.float64))
    # backbone codes live only on kept positions; off the mask the residual is x'
    bb = unpack_nibbles(out["bb_codes"])
    assert np.all(bb[~keep] == 0)
    assert np.array_equal(r[~keep], xp[~keep])
    # the backbone's scale equals the plain MXFP4 scale of x' (each group keeps its max)
    _, e_plain = mxfp4_quantize(xp)
    assert np.array_equal(out["bb_scales"].astype(np.int64) - 127, e_plain)
    # codes lie on the E2M1 grid: any nibble is valid; dequantised backbone equals q
    assert np.array_equal(mxfp4_dequantize(bb, out["bb_e"]).astype(np.float32), q)


def test_gamma_absorption_exact():
    rng = np.random.default_rng(0)
    x = bf16_round(rng.standard_normal((4, 64)).astype(np.float32) * 10)
    g = bf16_round(rng.uniform(0.5, 1.5, 64).astype(np.float32))
    xp = absorb_gamma(x, g)
    exact = bf16_to_f32(x).astype(np.float64) * bf16_to_f32(g).astype(np.float64)[None, :]
    assert np.array_equal(xp.astype(np.float64), exact)


def test_keep_all_reduces_to_plain_mxfp4():
    # with N = M the backbone is plain MXFP4 of x' and the residual is its error
    xb = _inputs(128, 2)
    out = prepare_ref(xb, None, 4, 4, keep_intermediates=True)
    codes, e = mxfp4_quantize(bf16_to_f32(xb))
    assert np.array_equal(out["bb_codes"], pack_nibbles(codes))
    assert np.array_equal(out["bb_scales"].astype(np.int64) - 127, e)
    q = mxfp4_dequantize(codes, e).astype(np.float32)
    assert np.array_equal(out["r"], (bf16_to_f32(xb) - q).astype(np.float32))


def test_prune_half_of_every_workload_row():
    w = workload_linear(T=8, K=512, O=32)
    out = prepare_ref(w["x"], None, 2, 4, keep_intermediates=True)
    assert out["keep"].mean() == 0.5
    d = workload_down_silu(T=4, K=256, O=16)
    out = prepare_ref(d["x"], None, 8, 16, keep_intermediates=True)
    assert out["keep"].mean() == 0.5


def test_rejects_non_finite_and_bad_shapes():
    x = bf16_round(np.array([[np.inf] + [0.0] * 31], np.float32))
    with pytest.raises(ValueError):
        prepare_ref(x, None, 2, 4)
    with pytest.raises(ValueError):
        prepare_ref(np.zeros((1, 48), np.uint16), None, 2, 4)


def test_residual_error_smaller_than_plain_fp4():
    # the decomposition should represent x' more accurately than one MXFP4 pass
    w = workload_linear(T=16, K=1024, O=8)
    x = bf16_to_f32(w["x"]).astype(np.float64)
    out = prepare_ref(w["x"], None, 2, 4, keep_intermediates=True)
    deq = (mxfp4_dequantize(out["bb_c"], out["bb_e"]) + mxfp4_dequantize(out["rs_c"], out["rs_e"]))
    codes, e = mxfp4_quantize(x.astype(np.float32))
    plain = mxfp4_dequantize(codes, e)
    assert np.linalg.norm(deq - x) < 0.5 * np.linalg.norm(plain - x)
