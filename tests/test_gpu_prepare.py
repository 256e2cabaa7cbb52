"""GPU parity of the prepare and plain-MXFP4 kernels against the CPU oracle.

Masks, codes and scales must match bit for bit. Cases span several workgroups
and a ragged tail, the edge cases of the method (ties, +-0, subnormals,
saturation, all-zero blocks, subnormal x*gamma products that take the exact
selection path), strided rows, and the full-size workload shapes (sampled rows).
"""

import numpy as np
import pytest

from oracle import prepare_ref, quantize_weight_ref
from synth import (adversarial_rows, bf16_round, bf16_to_f32, workload_down_silu, workload_linear,
                   workload_llama70b_decode, workload_llama8b_mlp, workload_qwen3_moe)
from gpu_util import assert_prepare_equal, bf16_to_gpu, to_np, w_codes_rows, w_scales_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _mixed_input(T, K, seed):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((T, K)) * rng.lognormal(0, 1.5, (T, 1))).astype(np.float32)
    base[:, rng.choice(K, max(1, K // 100), replace=False)] *= 50
    # small-integer rows: many exact ties inside groups
    base[: T // 4] = rng.integers(-3, 4, size=(T // 4, K)).astype(np.float32)
    return bf16_round(np.concatenate([base, adversarial_rows(K, seed)]))


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16)])
@pytest.mark.parametrize("with_gamma", [False, True])
@pytest.mark.parametrize("T,K", [(37, 352), (5, 32 * 16), (300, 1024)])
def test_prepare_small(sq, n, m, with_gamma, T, K):
    if K % m:
        pytest.skip("K must be a multiple of m")
    print(f"prepare small T={T} K={K} {n}:{m} gamma={with_gamma}", flush=True)
    xb = _mixed_input(T, K, seed=T + K)
    rng = np.random.default_rng(K)
    gamma = bf16_round(rng.uniform(0.5, 1.5, K).astype(np.float32)) if with_gamma else None
    want = prepare_ref(xb, gamma, n, m)
    got = sq.prepare(bf16_to_gpu(xb), None if gamma is None else bf16_to_gpu(gamma), n, m)
    assert_prepare_equal(got, want)


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16)])
def test_prepare_subnormal_gamma_products(sq, n, m):
    # x * gamma lands in the fp32 subnormal range with non-zero low mantissa
    # bits, which forces the exact (pairwise-rank) selection path; rows mix
    # such blocks with ordinary ones and with ties among subnormals.
    print(f"prepare subnormal products {n}:{m}", flush=True)
    T, K = 24, 256
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[::3] = rng.integers(-2, 3, size=(len(x[::3]), K))
    gamma = (rng.uniform(1, 2, K) * 2.0 ** -128).astype(np.float32)
    gamma[K // 2:] = rng.uniform(0.5, 1.5, K - K // 2)
    xb, gb = bf16_round(x), bf16_round(gamma)
    assert np.any(bf16_to_f32(gb) < 2.0 ** -126)
    want = prepare_ref(xb, gb, n, m)
    got = sq.prepare(bf16_to_gpu(xb), bf16_to_gpu(gb), n, m)
    assert_prepare_equal(got, want)


def test_prepare_strided_rows_single_block_and_no_mask(sq):
    import torch
    print("prepare strided / tiny / no-mask", flush=True)
    T, K, ld = 9, 96, 160
    rng = np.random.default_rng(2)
    wide = bf16_round((rng.standard_normal((T, ld)) * 3).astype(np.float32))
    xg = bf16_to_gpu(wide)[:, :K]
    assert xg.stride(0) == ld
    want = prepare_ref(wide[:, :K], None, 2, 4)
    assert_prepare_equal(sq.prepare(xg, None, 2, 4), want)
    got = sq.prepare(xg, None, 2, 4, with_mask=False)
    assert got.mask is None
    assert_prepare_equal(got, want)
    one = bf16_round(rng.standard_normal((1, 32)).astype(np.float32))
    assert_prepare_equal(sq.prepare(bf16_to_gpu(one), None, 8, 16), prepare_ref(one, None, 8, 16))
    # T = 0 is a no-op that returns empty outputs
    empty = sq.prepare(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), None, 2, 4)
    assert empty.bb_codes.shape == (1, 0, 64) and empty.bb_scales.shape == (1, 0, 4)


def test_prepare_deterministic(sq):
    print("prepare determinism", flush=True)
    xb = _mixed_input(200, 2048, 11)
    xg = bf16_to_gpu(xb)
    a = sq.prepare(xg, None, 8, 16)
    b = sq.prepare(xg, None, 8, 16)
    for f in ("bb_codes", "bb_scales", "res_codes", "res_scales", "mask"):
        assert np.array_equal(to_np(getattr(a, f)), to_np(getattr(b, f)))


def test_quantize_exhaustive_bf16(sq):
    # Every finite bf16 pattern, coded under six block exponents: each 32-block
    # holds an anchor 2^(E(v) + d) that fixes the block exponent and 31 test values.
    print("quantize exhaustive bf16", flush=True)
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(u)
    u = u[np.isfinite(f)]
    f = f[np.isfinite(f)]
    nz = f != 0
    e_of = np.zeros(len(f), np.int64)
    _, ex = np.frexp(np.abs(f[nz]).astype(np.float64))
    e_of[nz] = ex - 1
    blocks = []
    for d in range(6):
        anchor_e = e_of + d
        ok = (anchor_e <= 127) & (anchor_e >= -133)
        vals, ae = f[ok], anchor_e[ok]
        order = np.argsort(ae, kind="stable")
        vals, ae = vals[order], ae[order]
        # group values that share an anchor exponent into blocks of 31
        for a in np.unique(ae):
            v = vals[ae == a]
            pad = (-len(v)) % 31
            v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, 31)
            anchor = np.full((len(v), 1), np.ldexp(1.0, int(a)), np.float32)
            blocks.append(np.concatenate([anchor, v], axis=1))
    x = np.concatenate(blocks)
    rows = bf16_round(x)  # every entry is already bf16-exact
    assert np.array_equal(bf16_to_f32(rows), x)
    wc, ws = quantize_weight_ref(rows)
    got = sq.quantize_mxfp4(bf16_to_gpu(rows))
    assert np.array_equal(w_scales_rows(got.scales, ws.shape[1]), ws)
    assert np.array_equal(w_codes_rows(got.codes, wc.shape[1]), wc)


def test_quantize_weights_and_ragged(sq):
    print("quantize weights", flush=True)
    w = workload_linear(T=8, K=4096, O=4096)["w"]
    wc, ws = quantize_weight_ref(w)
    got = sq.quantize_mxfp4(bf16_to_gpu(w))
    assert np.array_equal(w_codes_rows(got.codes, wc.shape[1]), wc) and np.array_equal(w_scales_rows(got.scales, ws.shape[1]), ws)
    xb = _mixed_input(33, 160, 3)
    wc, ws = quantize_weight_ref(xb)
    got = sq.quantize_mxfp4(bf16_to_gpu(xb))
    assert np.array_equal(w_codes_rows(got.codes, wc.shape[1]), wc) and np.array_equal(w_scales_rows(got.scales, ws.shape[1]), ws)


def _rows_sample(T, count, seed):
    rng = np.random.default_rng(seed)
    if T <= count:
        return np.arange(T)
    return np.sort(np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), count - 2, replace=False)]))


@pytest.mark.parametrize("name", ["linear_128x4096", "llama8b_x", "down_silu_8of16", "down_silu_2of4",
                                  "qwen3_tokens", "llama70b_T64", "llama70b_T32", "llama70b_T8",
                                  "llama70b_T1"])
def test_prepare_workloads_full_size(sq, name):
    print(f"prepare workload {name}", flush=True)
    gamma = None
    if name == "linear_128x4096":
        x, n, m = workload_linear()["x"], 2, 4
    elif name == "llama8b_x":
        wl = workload_llama8b_mlp(with_weights=False)
        x, gamma, n, m = wl["x"], wl["gamma"], 2, 4
    elif name.startswith("down_silu"):
        x = workload_down_silu(with_weights=False)["x"]
        n, m = (8, 16) if name.endswith("8of16") else (2, 4)
    elif name == "qwen3_tokens":
        x, n, m = workload_qwen3_moe(with_weights=False)["x"], 2, 4
    else:
        T = int(name.split("_T")[1])
        x, n, m = workload_llama70b_decode(T, with_weights=False)["x"], 2, 4
    got = sq.prepare(bf16_to_gpu(x), None if gamma is None else bf16_to_gpu(gamma), n, m)
    rows = _rows_sample(x.shape[0], 192, seed=x.shape[1])
    want = prepare_ref(x[rows], gamma, n, m)
    assert_prepare_equal(got, want, rows=rows)
