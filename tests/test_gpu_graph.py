"""HIP graph capture of the chained MLP step, as the benchmark times it: the
library enqueues kernel launches only, so a captured step replays to the same
bits as the eager step. Each graph is replayed several times with eager work
and synchronisations between the replays (output buffers poisoned before each
replay), and every replay is compared with the eager result bit for bit."""

import numpy as np
import pytest

from synth import bf16_round
from gpu_util import bf16_to_gpu, to_np

pytestmark = pytest.mark.gpu

FIELDS = ("bb_codes", "bb_scales", "res_codes", "res_scales", "mask")


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _snapshot(bufs):
    out = {}
    for k, v in bufs.items():
        if hasattr(v, "bb_codes"):
            for f in FIELDS:
                out[f"{k}.{f}"] = to_np(getattr(v, f)).copy()
        else:
            out[k] = to_np(v).copy()
    return out


def _poison(bufs):
    for v in bufs.values():
        if hasattr(v, "bb_codes"):
            for f in FIELDS:
                getattr(v, f).fill_(0xA5)
        else:
            v.fill_(float("nan") if v.is_floating_point() else 7)


@pytest.mark.parametrize("T,H,I", [(300, 512, 384), (8, 4096, 2048), (2048, 4096, 14336)])
def test_captured_mlp_step_replays_bit_identical(sq, T, H, I):
    # (300, 512, 384): prepare_rms -> fused gate|up (128-row ring) -> down; (8, 4096, 2048): the decode tiles,
    # whose plan splits K (split kernels and their reduce inside the graph); (2048, 4096, 14336): the
    # Llama-3.1-8B step the benchmark times (a kernel that started before its predecessor ended would
    # read a half-written input)
    import torch
    from activation_sparsity_fp4_amd import _lib
    print(f"graph capture of the MLP step T={T} H={H} I={I}", flush=True)
    rng = np.random.default_rng(T + H)
    x = bf16_to_gpu(bf16_round((rng.standard_normal((T, H)) * rng.lognormal(0, 0.5, (T, 1))).astype(np.float32)))
    gamma = bf16_to_gpu(bf16_round(rng.uniform(0.5, 1.5, H).astype(np.float32)))
    w_gu = sq.quantize_mxfp4(bf16_to_gpu(bf16_round((rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32))))
    w_dn = sq.quantize_mxfp4(bf16_to_gpu(bf16_round((rng.standard_normal((H, I)) * 0.02).astype(np.float32))))
    if T <= 64:
        assert _lib.call("sharq_linear_workspace_bytes", T, H, I) > 0, "the decode shape must split K"
    bufs = {"p1": sq.prepare(x, gamma, 2, 4, rms_eps=1e-5)}
    bufs["p2"], _ = sq.linear_silu_prepare(bufs["p1"], w_gu, 2, 4)
    bufs["y"] = sq.linear(bufs["p2"], w_dn)

    def step():
        sq.prepare(x, gamma, 2, 4, out=bufs["p1"], rms_eps=1e-5)
        sq.linear_silu_prepare_into(bufs["p1"], w_gu, bufs["p2"], 2, 4)
        sq.linear(bufs["p2"], w_dn, out=bufs["y"])

    step()
    torch.cuda.synchronize()
    want = _snapshot(bufs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        _poison(bufs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(bufs)
        for k in want:
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), f"replay {rep}: {k} differs"
        # eager work between replays
        step()
        torch.cuda.synchronize()
