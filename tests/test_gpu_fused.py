"""GPU parity of the fused gate|up entry point (two-path GEMM -> silu(gate) * up
-> prepare) against the unfused chain linear -> silu_mul -> prepare, which the
other GPU tests check against the oracle.

The fused kernel runs the same MFMA sequence per output element as the plain
GEMM and the same SiLU and per-block prepare code, so h, codes, scales and
masks must match the unfused chain bit for bit. On sampled rows the fused
outputs are also checked against the oracle directly:
  - h on sampled columns against silu(g) * u of the oracle's float64 gate and
    up outputs (prepare_ref of x, quantize_weight_ref of the gate and up rows,
    linear_ref), within the tolerance that the Y bound implies for h
    (gpu_util.assert_h_close);
  - prepare_ref of the fused h reproduces the fused codes, scales and mask;
  - h is the correctly rounded silu(g) * u of the GPU's own GEMM output to
    one bf16 ulp.
"""

import numpy as np
import pytest

from oracle import linear_ref, prepare_ref, quantize_weight_ref, silu_mul_ref
from synth import bf16_round, workload_llama8b_mlp
from gpu_util import assert_bf16_close, assert_h_close, assert_prepare_equal, bf16_to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


FIELDS = ("bb_codes", "bb_scales", "res_codes", "res_scales", "mask")


def _inputs(T, I, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 0.5, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 200), replace=False)] *= 50
    w = (rng.standard_normal((2 * I, K)) * 0.02).astype(np.float32)
    return bf16_round(x), bf16_round(w)


def _check_fused(sq, x_bits, gamma_bits, w_bits, n, m, rows_sample):
    import torch
    T, K = x_bits.shape
    I = w_bits.shape[0] // 2
    p1 = sq.prepare(bf16_to_gpu(x_bits), None if gamma_bits is None else bf16_to_gpu(gamma_bits), 2, 4)
    w = sq.quantize_mxfp4(bf16_to_gpu(w_bits))
    # unfused chain
    y = sq.linear(p1, w)
    h_ref = sq.silu_mul(y)
    p2_ref = sq.prepare(h_ref, None, n, m)
    # fused, all outputs
    hp, h = sq.linear_silu_prepare(p1, w, n, m, with_h=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(h), to_np(h_ref)), "fused h differs from linear -> silu_mul"
    for f in FIELDS:
        assert np.array_equal(to_np(getattr(hp, f)), to_np(getattr(p2_ref, f))), f"fused {f} differs"
    # prepared output only, without the mask; h only
    hp2, h2 = sq.linear_silu_prepare(p1, w, n, m, with_h=False, with_mask=False)
    assert h2 is None and hp2.mask is None
    for f in FIELDS[:4]:
        assert np.array_equal(to_np(getattr(hp2, f)), to_np(getattr(p2_ref, f)))
    hp3, h3 = sq.linear_silu_prepare(p1, w, n, m, with_h=True, with_prepared=False)
    assert hp3 is None and np.array_equal(to_np(h3), to_np(h_ref))
    # oracle on sampled rows
    h_np = to_np(h)
    rows = rows_sample
    assert_prepare_equal(hp, prepare_ref(h_np[rows], None, n, m), rows=rows)
    assert_bf16_close(h_np[rows], silu_mul_ref(to_np(y)[rows], I))
    rng = np.random.default_rng(T + I)
    cols = np.unique(np.concatenate([[0, I - 1], rng.choice(I, min(I, 48), replace=False)]))
    check_h_against_oracle(h_np, x_bits, gamma_bits, w_bits[cols], w_bits[I + cols], rows, cols)


def check_h_against_oracle(h_np, x_bits, gamma_bits, w_gate, w_up, rows, cols):
    """The fused h on rows x cols against silu(g) * u of the oracle's float64
    gate and up outputs; w_gate / w_up are the bf16 weight rows of those h
    columns."""
    o1 = prepare_ref(x_bits[rows], gamma_bits, 2, 4)
    wc, ws = quantize_weight_ref(np.concatenate([w_gate, w_up]))
    y_ref, bound = linear_ref(o1["bb_codes"], o1["bb_scales"], o1["res_codes"], o1["res_scales"], wc, ws)
    nc = len(cols)
    assert_h_close(h_np[np.ix_(rows, cols)], y_ref[:, :nc], bound[:, :nc], y_ref[:, nc:], bound[:, nc:])


@pytest.mark.parametrize("T,I,K,n,m", [(300, 256, 512, 2, 4), (1, 128, 128, 2, 4), (130, 384, 1024, 8, 16),
                                       (2048, 4096, 512, 2, 4), (129, 128, 256, 8, 16), (20, 2048, 1024, 2, 4),
                                       (33, 2048, 1024, 8, 16), (64, 2048, 1024, 2, 4)])
def test_fused_matches_unfused(sq, T, I, K, n, m):
    # (2048, 4096): 512 tiles, the two-workgroups-per-CU kernel; T <= 32 and T <= 64 (without a K split
    # here) the 32- and 64-row decode tiles; the others the 4-stage ring
    print(f"fused gate|up T={T} I={I} K={K} {n}:{m}", flush=True)
    x, w = _inputs(T, I, K, seed=T + I + K)
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(1).choice(T, min(T, 24), replace=False)]))
    _check_fused(sq, x, None, w, n, m, rows)


def test_fused_llama8b_gate_up_full_size(sq):
    # the benchmark's fused stage: 2048 x 4096 -> gate|up 2 x 14336, gamma absorbed in the first prepare
    print("fused gate|up workload llama8b 2048x4096 -> 2x14336", flush=True)
    wl = workload_llama8b_mlp()
    rows = np.unique(np.concatenate([[0, 2047], np.random.default_rng(2).choice(2048, 24, replace=False)]))
    _check_fused(sq, wl["x"], wl["gamma"], wl["w_gu"], 2, 4, rows)


@pytest.mark.parametrize("T,I,K,n,m", [(1, 1024, 4096, 2, 4), (5, 512, 2048, 8, 16), (64, 1024, 4096, 2, 4),
                                       (200, 512, 4096, 8, 16)])
def test_fused_split_k_matches_split_chain(sq, T, I, K, n, m):
    # decode-sized T: the fused entry splits K as linear does (S = 4 .. 8 here) and sums, gates and
    # prepares in one more kernel; the chain is linear (same split plan) -> silu_mul -> prepare
    import torch
    from activation_sparsity_fp4_amd import _lib
    S_bytes = _lib.call("sharq_linear_silu_prepare_workspace_bytes", T, I, K)
    assert S_bytes > 0, "the shape must take the split-K path"
    assert S_bytes == _lib.call("sharq_linear_workspace_bytes", T, 2 * I, K), "the chain must split the same way"
    print(f"fused split-K T={T} I={I} K={K} {n}:{m} workspace {S_bytes}", flush=True)
    x, w = _inputs(T, I, K, seed=7 * T + I + K)
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(3).choice(T, min(T, 16), replace=False)]))
    _check_fused(sq, x, None, w, n, m, rows)


def test_fused_llama70b_decode_gate_up(sq):
    # the Llama-3.1-70B decode gate|up at T = 1 (2 x 28672 outputs, K = 8192): streamed whole on the
    # 32-row decode tile, as the plain GEMM runs it; against linear -> silu_mul -> prepare bit for bit.
    # Weights drawn on the GPU from a fixed seed.
    import torch
    from activation_sparsity_fp4_amd import _lib
    print("fused llama70b decode gate|up T=1", flush=True)
    g = torch.Generator(device="cuda").manual_seed(70)
    I, K = 28672, 8192
    assert _lib.call("sharq_linear_silu_prepare_workspace_bytes", 1, I, K) == 0, "no K split at this width"
    w_bf16 = (torch.randn(2 * I, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    w = sq.quantize_mxfp4(w_bf16)
    rng = np.random.default_rng(70)
    x = bf16_round((rng.standard_normal((1, K)) * 2).astype(np.float32))
    p1 = sq.prepare(bf16_to_gpu(x), None, 2, 4)
    y = sq.linear(p1, w)
    h_ref = sq.silu_mul(y)
    p2_ref = sq.prepare(h_ref, None, 2, 4)
    hp, h = sq.linear_silu_prepare(p1, w, 2, 4, with_h=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(h), to_np(h_ref))
    for f in FIELDS:
        assert np.array_equal(to_np(getattr(hp, f)), to_np(getattr(p2_ref, f))), f
    h_np = to_np(h)
    assert_prepare_equal(hp, prepare_ref(h_np, None, 2, 4))
    assert_bf16_close(h_np, silu_mul_ref(to_np(y), I))
    cols = np.unique(np.concatenate([[0, I - 1], rng.choice(I, 64, replace=False)]))
    idx = torch.from_numpy(cols).cuda()
    check_h_against_oracle(h_np, x, None, to_np(w_bf16[idx]), to_np(w_bf16[I + idx]), np.array([0]), cols)
