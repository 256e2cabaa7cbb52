"""GPU parity of the two-path FP4 GEMM against the oracle's fp64 product.

Inputs to the GEMM are the oracle's own prepare and weight-quantiser outputs
(uploaded), so every expected value comes from the oracle. Tolerance per
element: |Y_gpu - Y_ref| <= 1e-4 * sum_k |a_k w_k| + 1e-6.
Full-size workload shapes run in the same launch configuration the bench
times; their outputs are checked on sampled rows and columns.
"""

import numpy as np
import pytest

from oracle import linear_ref, prepare_ref, quantize_weight_ref
from synth import bf16_round, workload_down_silu, workload_linear, workload_llama8b_mlp
from gpu_util import (assert_prepare_equal, assert_y_close, bf16_to_gpu, oracle_prepared, to_np, u8_to_gpu,
                      w_codes_rows, w_scales_rows, w_to_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _random_problem(T, O, K, seed, n=2, m=4):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 1, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 40
    w = (rng.standard_normal((O, K)) * 0.02).astype(np.float32)
    p = prepare_ref(bf16_round(x), None, n, m)
    wc, ws = quantize_weight_ref(bf16_round(w))
    return p, wc, ws


@pytest.mark.parametrize("T,O,K", [(37, 70, 352), (300, 600, 1024), (1, 1, 32), (129, 257, 160),
                                   (128, 256, 128), (200, 513, 4096), (20, 700, 512), (32, 300, 256),
                                   (1, 256, 128), (48, 700, 512), (64, 256, 256)])
def test_linear_small(sq, T, O, K):
    # (20, 700, 512), (32, 300, 256), (1, 256, 128): the 32-row decode tile without a K split;
    # (48, 700, 512), (64, 256, 256): the 64-row one
    print(f"linear T={T} O={O} K={K}", flush=True)
    p, wc, ws = _random_problem(T, O, K, seed=T * 7 + O)
    y = sq.linear(oracle_prepared(p), w_to_gpu(wc, ws))
    y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    assert_y_close(to_np(y), y_ref, bound)


def test_linear_strided_output_and_zero_rows(sq):
    import torch
    print("linear ldy > O, T = 0", flush=True)
    T, O, K = 70, 96, 256
    p, wc, ws = _random_problem(T, O, K, seed=4)
    out = torch.full((T, O + 40), 7.0, dtype=torch.float32, device="cuda")[:, :O]
    sq.linear(oracle_prepared(p), w_to_gpu(wc, ws), out=out)
    y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    assert_y_close(to_np(out), y_ref, bound)
    full = to_np(out.as_strided((T, O + 40), (O + 40, 1)))
    assert np.all(full[:, O:] == 7.0)  # padding columns untouched
    G = sq.stages(K)
    e = sq.Prepared(torch.empty((G, 0, 64), dtype=torch.uint8, device="cuda"),
                    torch.empty((G, 0, 4), dtype=torch.uint8, device="cuda"),
                    torch.empty((G, 0, 64), dtype=torch.uint8, device="cuda"),
                    torch.empty((G, 0, 4), dtype=torch.uint8, device="cuda"), None, K)
    y0 = sq.linear(e, w_to_gpu(wc, ws))
    assert y0.shape == (0, O)


def test_linear_residual_only_and_backbone_only(sq):
    # zeroing one path's codes must leave exactly the other path's plain MXFP4 GEMM
    print("linear single paths", flush=True)
    T, O, K = 64, 128, 512
    p, wc, ws = _random_problem(T, O, K, seed=9)
    for zero in ("bb_codes", "res_codes"):
        q = dict(p)
        q[zero] = np.zeros_like(p[zero])
        y = sq.linear(oracle_prepared(q), w_to_gpu(wc, ws))
        y_ref, bound = linear_ref(q["bb_codes"], q["bb_scales"], q["res_codes"], q["res_scales"], wc, ws)
        assert_y_close(to_np(y), y_ref, bound)


def test_linear_deterministic(sq):
    print("linear determinism", flush=True)
    p, wc, ws = _random_problem(256, 512, 2048, seed=1)
    a = to_np(sq.linear(oracle_prepared(p), w_to_gpu(wc, ws)))
    b = to_np(sq.linear(oracle_prepared(p), w_to_gpu(wc, ws)))
    assert np.array_equal(a, b)


def test_linear_128x4096_full(sq):
    # single linear layer, 2:4: X [128 x 4096], W [4096 x 4096], every output checked
    print("linear workload 128x4096", flush=True)
    wl = workload_linear()
    p = prepare_ref(wl["x"], None, 2, 4)
    wc, ws = quantize_weight_ref(wl["w"])
    # GPU path end to end: prepare + weight quantiser + GEMM
    prep = sq.prepare(bf16_to_gpu(wl["x"]), None, 2, 4)
    wq = sq.quantize_mxfp4(bf16_to_gpu(wl["w"]))
    assert_prepare_equal(prep, p)
    assert np.array_equal(w_codes_rows(wq.codes, wc.shape[1]), wc) and np.array_equal(w_scales_rows(wq.scales, ws.shape[1]), ws)
    y = sq.linear(prep, wq)
    y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    assert_y_close(to_np(y), y_ref, bound)


def _sampled_linear_check(sq, x, gamma, n, m, w_bits, rows, cols):
    """GPU prepare + quantise + GEMM at full size; oracle on sampled rows/cols."""
    prep = sq.prepare(bf16_to_gpu(x), None if gamma is None else bf16_to_gpu(gamma), n, m)
    wq = sq.quantize_mxfp4(bf16_to_gpu(w_bits))
    y = sq.linear(prep, wq)
    p = prepare_ref(x[rows], gamma, n, m)
    assert_prepare_equal(prep, p, rows=rows)
    wc, ws = quantize_weight_ref(w_bits[cols])
    assert np.array_equal(w_codes_rows(wq.codes, wc.shape[1])[cols], wc)
    assert np.array_equal(w_scales_rows(wq.scales, ws.shape[1])[cols], ws)
    y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    assert_y_close(to_np(y)[np.ix_(rows, cols)], y_ref, bound)


def _sample(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, count, replace=False)]))


def test_llama8b_gate_up_full_size(sq):
    print("linear workload llama8b gate|up 2048x4096 -> 28672", flush=True)
    wl = workload_llama8b_mlp()
    _sampled_linear_check(sq, wl["x"], wl["gamma"], 2, 4, wl["w_gu"], _sample(2048, 48, 1), _sample(28672, 384, 2))


@pytest.mark.parametrize("n,m", [(8, 16), (2, 4)])
def test_down_proj_full_size(sq, n, m):
    print(f"linear workload down 2048x14336 -> 4096 {n}:{m}", flush=True)
    wl = workload_down_silu()
    _sampled_linear_check(sq, wl["x"], None, n, m, wl["w"], _sample(2048, 48, 3), _sample(4096, 384, 4))


def test_linear_big_tile_ragged(sq):
    # enough 256 x 256 tiles for the large-tile kernel, with a ragged last row
    # tile (2 rows) and a ragged last column tile; sampled rows and columns
    # include both edges
    print("linear 256x256 tiles, ragged: 2050 x 1024 -> 22000", flush=True)
    T, K, O = 2050, 1024, 22000
    rng = np.random.default_rng(77)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 0.5, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, 8, replace=False)] *= 50
    w = (rng.standard_normal((O, K)) * 0.02).astype(np.float32)
    rows = np.unique(np.concatenate([_sample(T, 40, 5), [2046, 2047, 2048, 2049]]))
    cols = np.unique(np.concatenate([_sample(O, 300, 6), np.arange(O - 40, O), np.arange(21760, 21790)]))
    _sampled_linear_check(sq, bf16_round(x), None, 2, 4, bf16_round(w), rows, cols)
