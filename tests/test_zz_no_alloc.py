"""The scratch-free two-path GEMM (sharq_linear_scratchfree), called through
the C ABI, against the existing split-K entry point sharq_linear_ws with a
caller-owned workspace: the same split plan and kernels, so the outputs must
be bit-identical; sampled columns are also checked against the oracle. Two
calls in a row, the second with a smaller input (the static array keeps the
first call's partials), then one that plans no split."""

import numpy as np
import pytest

from oracle import linear_ref, prepare_ref, quantize_weight_ref
from synth import bf16_round
from gpu_util import assert_y_close, bf16_to_gpu, oracle_prepared, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _call(lib_call, name, p, w, T, O, K, y, *extra):
    import torch
    return lib_call(name, p.bb_codes.data_ptr(), p.bb_scales.data_ptr(), p.res_codes.data_ptr(),
                    p.res_scales.data_ptr(), w.codes.data_ptr(), w.scales.data_ptr(), T, O, K, y.data_ptr(), O,
                    *extra, torch.cuda.current_stream().cuda_stream)


def test_scratchfree_matches_linear_ws(sq):
    import torch
    from activation_sparsity_fp4_amd import _lib
    O, K = 8192, 28672
    g = torch.Generator(device="cuda").manual_seed(77)
    w_bf = (torch.randn(O, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    w = sq.quantize_mxfp4(w_bf)
    rng = np.random.default_rng(77)
    cols = np.unique(np.concatenate([[0, O - 1], rng.choice(O, 64, replace=False)]))
    wc, ws = quantize_weight_ref(to_np(w_bf[torch.from_numpy(cols).cuda()]))
    for T in (64, 8, 3):  # a large split, a smaller one (stale partials in the array), then a smaller still
        need = _lib.call("sharq_linear_workspace_bytes", T, O, K)
        print(f"scratch-free linear T={T} O={O} K={K} partials {need} bytes", flush=True)
        assert 0 < need <= _lib.SCRATCHFREE_MAX_BYTES
        x = bf16_round((rng.standard_normal((T, K)) * rng.lognormal(0, 0.5, (T, 1))).astype(np.float32))
        pr = prepare_ref(x, None, 2, 4)
        p = oracle_prepared(pr)
        y_sf = torch.full((T, O), float("nan"), dtype=torch.float32, device="cuda")
        y_ws = torch.full((T, O), float("nan"), dtype=torch.float32, device="cuda")
        work = torch.empty(need, dtype=torch.uint8, device="cuda")
        assert _call(_lib.call, "sharq_linear_scratchfree", p, w, T, O, K, y_sf) == _lib.SHARQ_OK
        assert _call(_lib.call, "sharq_linear_ws", p, w, T, O, K, y_ws, work.data_ptr(), need) == _lib.SHARQ_OK
        torch.cuda.synchronize()
        a, b = to_np(y_sf), to_np(y_ws)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "scratch-free output differs from linear_ws"
        y_ref, bound = linear_ref(pr["bb_codes"], pr["bb_scales"], pr["res_codes"], pr["res_scales"], wc, ws)
        assert_y_close(a[:, cols], y_ref, bound)


def test_scratchfree_without_split_and_refusal(sq):
    """A shape whose plan does not split runs as sharq_linear; a shape whose
    partials exceed the array is refused before any launch."""
    import torch
    from activation_sparsity_fp4_amd import _lib
    T, O, K = 1024, 2048, 256
    assert _lib.call("sharq_linear_workspace_bytes", T, O, K) == 0
    print(f"scratch-free linear T={T} O={O} K={K} no split", flush=True)
    rng = np.random.default_rng(5)
    x = bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    wb = bf16_round((rng.standard_normal((O, K)) * 0.02).astype(np.float32))
    w = sq.quantize_mxfp4(bf16_to_gpu(wb))
    p = sq.prepare(bf16_to_gpu(x), None, 2, 4)
    y_sf = torch.empty((T, O), dtype=torch.float32, device="cuda")
    assert _call(_lib.call, "sharq_linear_scratchfree", p, w, T, O, K, y_sf) == _lib.SHARQ_OK
    y = sq.linear(p, w)
    y_b = sq.linear_scratchfree(p, w, torch.empty((T, O), dtype=torch.float32, device="cuda"))  # the binding
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y_sf).view(np.uint32), to_np(y).view(np.uint32))
    assert np.array_equal(to_np(y_b).view(np.uint32), to_np(y).view(np.uint32))
    Tb, Ob, Kb = 320, 8192, 28672
    assert _lib.call("sharq_linear_workspace_bytes", Tb, Ob, Kb) > _lib.SCRATCHFREE_MAX_BYTES
    assert _lib.call("sharq_linear_scratchfree", 16, 16, 16, 16, 16, 16, Tb, Ob, Kb, 16, Ob,
                     torch.cuda.current_stream().cuda_stream) == _lib.SHARQ_ESCRATCH
