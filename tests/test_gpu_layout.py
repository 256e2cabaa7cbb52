"""GPU layout conversion between the canonical row-major block-FP4 layout and
the stage-major one: bit for bit against a NumPy relayout for MXFP4 (32-entry
scale blocks) and NVFP4 (16-entry), with a partial last stage, round trips,
and a linear layer run on a weight packed from the oracle's row-major output."""

import numpy as np
import pytest

from oracle import linear_ref, prepare_ref, quantize_weight_ref
from synth import bf16_round
from gpu_util import (assert_y_close, bf16_to_gpu, codes_stage_major, oracle_prepared, stage_major, to_np,
                      u8_to_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def scales_stage_major(s_rows, per_stage):
    """Row-major scale bytes [R, K/B] -> [G, R, per_stage], zero past K."""
    R, kb = s_rows.shape
    G = (kb + per_stage - 1) // per_stage
    pad = np.zeros((R, per_stage * G), dtype=np.uint8)
    pad[:, :kb] = s_rows
    return np.ascontiguousarray(pad.reshape(R, G, per_stage).transpose(1, 0, 2))


@pytest.mark.parametrize("R,K", [(37, 352), (256, 128), (5, 160), (300, 4096), (1, 32)])
@pytest.mark.parametrize("block", [32, 16])
def test_pack_and_unpack(sq, R, K, block):
    print(f"layout R={R} K={K} block={block}", flush=True)
    rng = np.random.default_rng(R * 31 + K + block)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (R, K // block), dtype=np.uint8)
    if block == 32:
        t = sq.pack_mxfp4(u8_to_gpu(codes), u8_to_gpu(scales), K)
        assert np.array_equal(to_np(t.scales), stage_major(scales))
    else:
        t = sq.pack_nvfp4(u8_to_gpu(codes), u8_to_gpu(scales), K, 0.5)
        assert np.array_equal(to_np(t.scales), scales_stage_major(scales, 8))
    assert np.array_equal(to_np(t.codes), codes_stage_major(codes))
    c2, s2 = sq.unpack_stage_major(t.codes, t.scales, K)
    assert np.array_equal(to_np(c2), codes) and np.array_equal(to_np(s2), scales)


def test_linear_on_a_packed_weight(sq):
    """A weight quantised elsewhere in the canonical layout (here by the
    oracle), packed on the GPU, then used by the two-path GEMM."""
    print("linear on packed weight", flush=True)
    rng = np.random.default_rng(8)
    T, K, O = 70, 384, 200
    x = bf16_round((rng.standard_normal((T, K)) * 2).astype(np.float32))
    wb = bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32))
    p = prepare_ref(x, None, 2, 4)
    wc, ws = quantize_weight_ref(wb)
    w = sq.pack_mxfp4(u8_to_gpu(wc), u8_to_gpu(ws), K)
    y = sq.linear(oracle_prepared(p), w)
    y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    assert_y_close(to_np(y), y_ref, bound)
    # and the library's own quantiser gives the same packed weight
    wq = sq.quantize_mxfp4(bf16_to_gpu(wb))
    assert np.array_equal(to_np(wq.codes), to_np(w.codes)) and np.array_equal(to_np(wq.scales), to_np(w.scales))


@pytest.mark.parametrize("T,K,n,m,with_gamma", [(37, 352, 2, 4, False), (300, 1024, 8, 16, True),
                                                  (2048, 4096, 2, 4, True), (64, 8192, 8, 16, False)])
def test_prepare_output_in_canonical_layout(sq, T, K, n, m, with_gamma):
    """The library's own prepare output, taken back to the canonical row-major
    layout by sharq_unpack_stage_major on the GPU, equals prepare_ref's
    canonical arrays byte for byte; the same for sharq_quantize_mxfp4 against
    quantize_weight_ref."""
    print(f"prepare -> unpack_stage_major T={T} K={K} {n}:{m} gamma={with_gamma}", flush=True)
    rng = np.random.default_rng(T + K + n)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 0.5, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 200), replace=False)] *= 50
    x = bf16_round(x)
    gamma = bf16_round(rng.uniform(0.5, 1.5, K).astype(np.float32)) if with_gamma else None
    p = sq.prepare(bf16_to_gpu(x), None if gamma is None else bf16_to_gpu(gamma), n, m)
    want = prepare_ref(x, gamma, n, m)
    for path in ("bb", "res"):
        c_rm, s_rm = sq.unpack_stage_major(getattr(p, f"{path}_codes"), getattr(p, f"{path}_scales"), K)
        assert np.array_equal(to_np(c_rm), want[f"{path}_codes"]), f"{path} codes"
        assert np.array_equal(to_np(s_rm), want[f"{path}_scales"]), f"{path} scales"
    assert np.array_equal(to_np(p.mask), want["mask"])
    O = 96
    wb = bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32))
    wq = sq.quantize_mxfp4(bf16_to_gpu(wb))
    wc, ws = quantize_weight_ref(wb)
    c_rm, s_rm = sq.unpack_stage_major(wq.codes, wq.scales, K)
    assert np.array_equal(to_np(c_rm), wc) and np.array_equal(to_np(s_rm), ws)
