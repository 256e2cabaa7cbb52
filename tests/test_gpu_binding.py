"""The binding refuses caller-supplied output buffers that do not fit the
result (wrong shape, dtype or stride) before any kernel is launched, so a
too-small buffer can never be written past its end."""

import numpy as np
import pytest

from synth import bf16_round
from gpu_util import bf16_to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def test_output_buffers_are_checked(sq):
    import torch
    print("binding output checks", flush=True)
    rng = np.random.default_rng(0)
    T, K, O = 64, 256, 128
    x = bf16_to_gpu(bf16_round(rng.standard_normal((T, K)).astype(np.float32)))
    w = bf16_to_gpu(bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32)))
    p = sq.prepare(x)
    wq = sq.quantize_mxfp4(w)
    f32 = dict(dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        sq.linear(p, wq, out=torch.empty((T - 1, O), **f32))          # too few rows
    with pytest.raises(ValueError):
        sq.linear(p, wq, out=torch.empty((T, 2 * O), **f32)[:, ::2])  # column stride 2
    with pytest.raises(TypeError):
        sq.linear(p, wq, out=torch.empty((T, O), dtype=torch.float16, device="cuda"))
    small = sq.prepare(x[: T // 2])
    with pytest.raises(ValueError):
        sq.prepare(x, out=small)                                      # out for fewer rows
    with pytest.raises(ValueError):
        sq.quantize_mxfp4(w, out=sq.quantize_mxfp4(w[: O // 2]))
    with pytest.raises(ValueError):
        sq.silu_mul(torch.zeros((T, 2 * O), **f32), out=torch.empty((T, O - 8), dtype=torch.bfloat16, device="cuda"))
    seg = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    wg = sq.MXFP4(wq.codes[None].contiguous(), wq.scales[None].contiguous(), K)
    with pytest.raises(ValueError):
        sq.linear_grouped(p, wg, seg, out=torch.empty((T, 2 * O), **f32)[:, :O])  # not contiguous
    pn = sq.prepare_nvfp4(x, 0.01)
    wn = sq.quantize_nvfp4(w, 1e-4)
    with pytest.raises(ValueError):
        sq.linear_nvfp4(pn, wn, out=torch.empty((T, O - 1), **f32))
    with pytest.raises(ValueError):
        sq.prepare_nvfp4(x, 0.01, out=sq.prepare_nvfp4(x[: T // 2], 0.01))
    # gamma must hold exactly K entries (the kernels read K of them)
    g_short = bf16_to_gpu(bf16_round(np.ones(K - 32, dtype=np.float32)))
    with pytest.raises(ValueError):
        sq.prepare(x, g_short)
    with pytest.raises(ValueError):
        sq.prepare(x, g_short, rms_eps=1e-5)
    with pytest.raises(ValueError):
        sq.prepare_nvfp4(x, 0.01, g_short)
    # well-formed buffers still work
    y = sq.linear(p, wq, out=torch.empty((T, O), **f32))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
