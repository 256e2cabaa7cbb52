"""GPU parity of the split-K two-path GEMM (sharq_linear_ws) used for problems
with too few output tiles to fill the GPU: decode-sized T and, for long K,
mid-sized T (several 128-row tiles, ragged rows and columns, split counts that
are not powers of two). Against the oracle's fp64 product to the GEMM
tolerance, bitwise repeatable, and with one workspace reused across shapes."""

import numpy as np
import pytest

from oracle import linear_ref, prepare_ref, quantize_weight_ref
from synth import bf16_round
from gpu_util import assert_y_close, oracle_prepared, to_np, w_to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _problem(T, O, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 1, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 40
    w = (rng.standard_normal((O, K)) * 0.02).astype(np.float32)
    p = prepare_ref(bf16_round(x), None, 2, 4)
    wc, ws = quantize_weight_ref(bf16_round(w))
    return p, wc, ws


@pytest.mark.parametrize("T,O,K", [(1, 8192, 4096), (5, 1000, 2048), (64, 2048, 8192), (12, 700, 3072),
                                   (3, 4096, 8192), (300, 1024, 4096), (500, 1000, 8192), (130, 3000, 4096),
                                   (65, 2048, 8192), (257, 1024, 8192)])
def test_split_k_matches_oracle_and_repeats(sq, T, O, K):
    from activation_sparsity_fp4_amd import _lib
    print(f"split-K T={T} O={O} K={K}", flush=True)
    assert _lib.call("sharq_linear_workspace_bytes", T, O, K) > 0, "shape expected to split"
    p, wc, ws = _problem(T, O, K, seed=T * 3 + O)
    prep, w = oracle_prepared(p), w_to_gpu(wc, ws)
    y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
    a = to_np(sq.linear(prep, w))
    b = to_np(sq.linear(prep, w))
    assert np.array_equal(a, b), "split-K result changed between calls"
    assert_y_close(a, y_ref, bound)
    c = to_np(sq.linear(prep, w, split_k=False))
    assert_y_close(c, y_ref, bound)


def test_split_k_workspace_shared_across_shapes(sq):
    # Different shapes (tile and split counts) one after another on one cached
    # workspace, whose contents each call overwrites.
    print("split-K workspace reuse", flush=True)
    probs = [(1, 2048, 4096, 1), (16, 16640, 2048, 2), (70, 512, 1024, 3), (1, 2048, 4096, 1),
             (16, 16640, 2048, 2)]
    seen = {}
    for T, O, K, seed in probs:
        p, wc, ws = _problem(T, O, K, seed)
        y = to_np(sq.linear(oracle_prepared(p), w_to_gpu(wc, ws)))
        y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
        assert_y_close(y, y_ref, bound)
        if seed in seen:
            assert np.array_equal(seen[seed], y)
        seen[seed] = y


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_llama70b_decode_shapes_full_size(sq, T):
    # the benchmark's decode GEMMs at full size, in the launch configuration it times (split K, 32- and
    # 64-row decode tiles): gate|up 2 x 28672 x 8192 and down 8192 x 28672, against the oracle on sampled
    # output columns (weights drawn on the GPU from a fixed seed; the sampled rows are quantised by the oracle)
    import torch
    from synth import workload_llama70b_decode
    print(f"llama70b decode full size T={T}", flush=True)
    wl = workload_llama70b_decode(T, with_weights=False)
    H, I = wl["hidden"], wl["inter"]
    g = torch.Generator(device="cuda").manual_seed(700 + T)
    for O, K, seed in ((2 * I, H, 1), (H, I, 2)):
        w_bf = (torch.randn(O, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        wq = sq.quantize_mxfp4(w_bf)
        rng = np.random.default_rng(seed + T)
        if K == H:
            x = wl["x"]
        else:
            x = bf16_round((rng.standard_normal((T, K)) * 0.5).astype(np.float32))
        p = prepare_ref(x, None, 2, 4)
        y = to_np(sq.linear(oracle_prepared(p), wq))
        cols = np.unique(np.concatenate([[0, O - 1], rng.choice(O, 96, replace=False)]))
        w_rows = to_np(w_bf[torch.from_numpy(cols).cuda().long()])
        wc, ws = quantize_weight_ref(w_rows)
        y_ref, bound = linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
        assert_y_close(y[:, cols], y_ref, bound)
