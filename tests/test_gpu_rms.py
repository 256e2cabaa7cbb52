"""GPU parity of the prepare operator with the whole RMSNorm absorbed
(sharq_prepare_rms): the per-row scales and every output bit for bit against
the oracle, on ragged shapes, block counts that are not powers of two, rows of
extreme magnitude, both N:M patterns, with and without gamma, and the
benchmark's full-size input."""

import numpy as np
import pytest

from oracle import prepare_ref
from synth import bf16_round, workload_llama8b_mlp
from gpu_util import assert_prepare_equal, bf16_to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _check(sq, x, g, n, m, eps, rows=None):
    got = sq.prepare(bf16_to_gpu(x), None if g is None else bf16_to_gpu(g), n, m, rms_eps=eps)
    xs = x if rows is None else x[rows]
    want = prepare_ref(xs, g, n, m, rms_eps=eps)
    r = to_np(got.rms_scale)
    r = r if rows is None else r[rows]
    bad = np.flatnonzero(r.view(np.uint32) != want["rms_scale"].view(np.uint32))
    assert bad.size == 0, f"rms scale differs on {bad.size} rows, first {bad[0]}: {r[bad[0]]} vs {want['rms_scale'][bad[0]]}"
    assert_prepare_equal(got, want, rows=rows)


@pytest.mark.parametrize("T,K,n,m,gamma", [(37, 352, 2, 4, True), (300, 1024, 8, 16, False), (1, 32, 2, 4, False),
                                           (129, 96, 8, 16, True), (64, 4128, 2, 4, True), (20, 8192, 8, 16, True),
                                           (6, 65568, 2, 4, False), (5, 131072, 8, 16, True)])
def test_prepare_rms_small(sq, T, K, n, m, gamma):
    # K = 65568 and 131072: 2049 and 4096 blocks per row, 3 and 4 rounds of the row-sum tree (the last the maximum)
    print(f"prepare rms T={T} K={K} {n}:{m} gamma={gamma}", flush=True)
    rng = np.random.default_rng(T * 31 + K)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 2, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 60
    g = bf16_round(rng.uniform(0.5, 1.5, K).astype(np.float32)) if gamma else None
    _check(sq, bf16_round(x), g, n, m, 1e-5)


def test_prepare_rms_extreme_rows(sq):
    print("prepare rms extreme rows", flush=True)
    rng = np.random.default_rng(3)
    K = 256
    rows = [np.zeros(K), np.full(K, 1e-38), np.full(K, 3e38), rng.standard_normal(K) * 1e-30,
            rng.standard_normal(K) * 1e30, np.concatenate([[1e20], np.zeros(K - 1)]),
            np.where(np.arange(K) % 2 == 0, 1.0, -1.0) * 2.0 ** -126]
    x = bf16_round(np.stack(rows).astype(np.float32))
    for eps in (1e-5, 1e-12, 1.0):
        _check(sq, x, None, 2, 4, eps)
        _check(sq, x, bf16_round(rng.uniform(0.5, 1.5, K).astype(np.float32)), 8, 16, eps)


def test_prepare_rms_llama8b_full_size(sq):
    print("prepare rms workload llama8b x 2048x4096", flush=True)
    wl = workload_llama8b_mlp(with_weights=False)
    rows = np.unique(np.concatenate([[0, 2047], np.random.default_rng(4).choice(2048, 200, replace=False)]))
    _check(sq, wl["x"], wl["gamma"], 2, 4, 1e-5, rows=rows)
