"""GPU parity of the NVFP4 path (prepare, weight quantiser, two-path GEMM)
against the CPU oracle: codes, E4M3 scales and masks bit for bit, Y within
1e-4 * sum|a w| + 1e-6. Cases span several workgroups, ragged row and column
tails, a partial last K stage, the edge cases of the block coding (ties,
signed zeros, subnormals, huge values, saturated and zero block scales), and
the Llama-3.1-8B down projection at full size on sampled rows and columns."""

import numpy as np
import pytest

from oracle import (linear_nvfp4_ref, prepare_nvfp4_ref, quantize_weight_nvfp4_ref, tensor_scale_from_amax)
from synth import adversarial_rows, bf16_round, bf16_to_f32, workload_down_silu
from gpu_util import assert_y_close, bf16_to_gpu, codes_row_major, codes_stage_major, to_np, u8_to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def nv_scales_stage_major(s_rows):
    """Row-major E4M3 bytes [R, K/16] -> the library's [ceil(K/128), R, 8] (zero past K)."""
    s_rows = np.asarray(s_rows, dtype=np.uint8)
    R, kb = s_rows.shape
    G = (kb + 7) // 8
    pad = np.zeros((R, 8 * G), dtype=np.uint8)
    pad[:, :kb] = s_rows
    return np.ascontiguousarray(pad.reshape(R, G, 8).transpose(1, 0, 2))


def nv_scales_row_major(s_stage, kblocks):
    """[G, R, 8] -> [R, K/16]; the padding bytes must be zero."""
    s_stage = np.asarray(s_stage, dtype=np.uint8)
    G, R, _ = s_stage.shape
    flat = s_stage.transpose(1, 0, 2).reshape(R, 8 * G)
    assert not flat[:, kblocks:].any(), "scale padding bytes must be zero"
    return flat[:, :kblocks]


def assert_nv_prepare_equal(got, want, rows=None):
    for name in ("bb_codes", "bb_scales", "res_codes", "res_scales", "mask"):
        g = getattr(got, name)
        if g is None:
            continue
        g = to_np(g)
        if name.endswith("scales"):
            g = nv_scales_row_major(g, want[name].shape[1])
        elif name.endswith("codes"):
            g = codes_row_major(g, want[name].shape[1])
        if rows is not None:
            g = g[rows]
        w = want[name]
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            r, c = bad[0]
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at row {r} col {c}: "
                                 f"gpu {g[r, c]:#x} oracle {w[r, c]:#x}")


def oracle_nv_prepared(sq, out, s_a):
    K = 2 * out["bb_codes"].shape[1]
    return sq.NVPrepared(u8_to_gpu(codes_stage_major(out["bb_codes"])), u8_to_gpu(nv_scales_stage_major(out["bb_scales"])),
                         u8_to_gpu(codes_stage_major(out["res_codes"])),
                         u8_to_gpu(nv_scales_stage_major(out["res_scales"])), None, K, float(s_a))


def oracle_nv_weight(sq, wc, ws, s_w):
    return sq.NVFP4(u8_to_gpu(codes_stage_major(wc)), u8_to_gpu(nv_scales_stage_major(ws)), 2 * wc.shape[1],
                    float(s_w))


def _mixed_input(T, K, seed):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((T, K)) * rng.lognormal(0, 1.5, (T, 1))).astype(np.float32)
    base[:, rng.choice(K, max(1, K // 100), replace=False)] *= 50
    base[: T // 4] = rng.integers(-3, 4, size=(T // 4, K)).astype(np.float32)  # exact ties
    return bf16_round(np.concatenate([base, adversarial_rows(K, seed)]))


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16)])
@pytest.mark.parametrize("with_gamma", [False, True])
@pytest.mark.parametrize("T,K", [(37, 352), (300, 1024), (5, 160)])
def test_prepare_nvfp4_small(sq, n, m, with_gamma, T, K):
    print(f"nvfp4 prepare T={T} K={K} {n}:{m} gamma={with_gamma}", flush=True)
    xb = _mixed_input(T, K, seed=T + K)
    rng = np.random.default_rng(K)
    gamma = bf16_round(rng.uniform(0.5, 1.5, K).astype(np.float32)) if with_gamma else None
    finite = bf16_to_f32(xb)
    amax = float(np.abs(finite[np.isfinite(finite)]).max())
    # the usual tensor scale, a neutral one, one that saturates block scales and one that zeroes them
    for s_a in (tensor_scale_from_amax(amax), 1.0, 2.0 ** -20, 1e3):
        want = prepare_nvfp4_ref(xb, gamma, n, m, s_a)
        got = sq.prepare_nvfp4(bf16_to_gpu(xb), s_a, None if gamma is None else bf16_to_gpu(gamma), n, m)
        assert_nv_prepare_equal(got, want)


def test_quantize_nvfp4(sq):
    print("nvfp4 weight quantiser", flush=True)
    rng = np.random.default_rng(21)
    for O, K in ((70, 384), (256, 160), (3, 32)):
        wb = bf16_round((rng.standard_normal((O, K)) * rng.lognormal(-4, 1, (O, 1))).astype(np.float32))
        s_w = tensor_scale_from_amax(np.abs(bf16_to_f32(wb)).max())
        wc, ws = quantize_weight_nvfp4_ref(wb, s_w)
        got = sq.quantize_nvfp4(bf16_to_gpu(wb), s_w)
        assert np.array_equal(codes_row_major(to_np(got.codes), wc.shape[1]), wc)
        assert np.array_equal(nv_scales_row_major(to_np(got.scales), ws.shape[1]), ws)


@pytest.mark.parametrize("T,O,K", [(200, 300, 384), (128, 256, 512), (33, 70, 160), (1, 256, 128), (257, 513, 256)])
def test_linear_nvfp4_oracle_inputs(sq, T, O, K):
    """The GEMM alone, on oracle-prepared operands (several tiles, ragged T and
    O, a partial last stage)."""
    print(f"nvfp4 linear T={T} O={O} K={K}", flush=True)
    rng = np.random.default_rng(T * 7 + O + K)
    x = bf16_round((rng.standard_normal((T, K)) * rng.lognormal(0, 1, (T, 1))).astype(np.float32))
    s_a = tensor_scale_from_amax(np.abs(bf16_to_f32(x)).max())
    p = prepare_nvfp4_ref(x, None, 2, 4, s_a)
    wb = bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32))
    s_w = tensor_scale_from_amax(np.abs(bf16_to_f32(wb)).max())
    wc, ws = quantize_weight_nvfp4_ref(wb, s_w)
    y = sq.linear_nvfp4(oracle_nv_prepared(sq, p, s_a), oracle_nv_weight(sq, wc, ws, s_w))
    y_ref, bound = linear_nvfp4_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], s_a, wc, ws, s_w)
    assert_y_close(to_np(y), y_ref, bound)


def test_linear_nvfp4_strided_output(sq):
    import torch
    print("nvfp4 linear strided output", flush=True)
    rng = np.random.default_rng(3)
    T, O, K = 64, 256, 256
    x = bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    p = prepare_nvfp4_ref(x, None, 8, 16, 0.01)
    wb = bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32))
    wc, ws = quantize_weight_nvfp4_ref(wb, 1e-5)
    big = torch.full((T, O + 64), 7.0, dtype=torch.float32, device="cuda")
    sq.linear_nvfp4(oracle_nv_prepared(sq, p, 0.01), oracle_nv_weight(sq, wc, ws, 1e-5), out=big[:, :O])
    y_ref, bound = linear_nvfp4_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], 0.01, wc, ws,
                                    1e-5)
    assert_y_close(to_np(big[:, :O]), y_ref, bound)
    assert torch.all(big[:, O:] == 7.0), "columns past O were written"


def test_nvfp4_llama8b_down_full_size(sq):
    """The Llama-3.1-8B down projection at full size (2048 x 14336 -> 4096,
    8:16) in the benchmark's launch configuration: GPU prepare, quantiser and
    GEMM; the oracle recomputes sampled rows of the prepare, sampled weight
    rows, and Y on their crossing."""
    import torch
    print("nvfp4 llama8b down full size", flush=True)
    wl = workload_down_silu()
    xb, w, n, m = wl["x"], wl["w"], wl["n"], wl["m"]
    T, K = xb.shape
    O = w.shape[0]
    s_a = tensor_scale_from_amax(np.abs(bf16_to_f32(xb)).max())
    s_w = tensor_scale_from_amax(np.abs(bf16_to_f32(w)).max())
    p = sq.prepare_nvfp4(bf16_to_gpu(xb), s_a, None, n, m)
    wq = sq.quantize_nvfp4(bf16_to_gpu(w), s_w)
    y = to_np(sq.linear_nvfp4(p, wq))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 6, replace=False)]))
    cols = np.unique(np.concatenate([[0, O - 1], rng.choice(O, 14, replace=False)]))
    want = prepare_nvfp4_ref(xb[rows], None, n, m, s_a)
    assert_nv_prepare_equal(p, want, rows=rows)
    wc, ws = quantize_weight_nvfp4_ref(w[cols], s_w)
    assert np.array_equal(codes_row_major(to_np(wq.codes), K // 2)[cols], wc)
    assert np.array_equal(nv_scales_row_major(to_np(wq.scales), K // 16)[cols], ws)
    y_ref, bound = linear_nvfp4_ref(want["bb_codes"], want["bb_scales"], want["res_codes"], want["res_scales"], s_a,
                                    wc, ws, s_w)
    assert_y_close(y[np.ix_(rows, cols)], y_ref, bound)
