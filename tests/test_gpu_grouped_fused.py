"""GPU parity of the grouped fused gate|up entry point (per-expert two-path
GEMM -> silu(gate) * up -> prepare) against the unfused chain
linear_grouped -> silu_mul -> prepare, which the other GPU tests check against
the oracle.

The fused kernel runs the grouped GEMM's MFMA sequence per output element and
the same SiLU and per-block prepare code, so h, codes, scales and masks must
match the chain bit for bit. On sampled pairs the fused outputs are also
checked against the oracle directly:
  - h on sampled columns against silu(g) * u of the oracle's float64 gate and
    up outputs for the pair's token and expert (linear_ref), within the
    tolerance the Y bound implies for h (gpu_util.assert_h_close);
  - prepare_ref of the fused h reproduces the fused codes, scales and mask;
  - h is the correctly rounded silu(g) * u of the chain's GEMM output to one
    bf16 ulp.
"""

import numpy as np
import pytest

from oracle import linear_ref, prepare_ref, quantize_weight_ref, silu_mul_ref
from synth import bf16_round, moe_routing, workload_qwen3_moe
from gpu_util import (assert_bf16_close, assert_h_close, assert_prepare_equal, bf16_to_gpu, i32_to_gpu,
                      oracle_prepared, to_np, w_to_gpu)

pytestmark = pytest.mark.gpu

FIELDS = ("bb_codes", "bb_scales", "res_codes", "res_scales", "mask")


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _check_h_oracle(h_np, pairs, seg, a_rows, I, prep_rows, w_rows, seed):
    """h of sampled pairs and columns against silu(g) * u of the oracle's gate
    and up outputs. prep_rows(src) -> prepare_ref dict of those source rows;
    w_rows(e, rows) -> (codes, scales) of expert e's weight rows, row-major."""
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([[0, I - 1], rng.choice(I, min(I, 32), replace=False)]))
    nc = len(cols)
    e_of = np.searchsorted(seg, pairs, side="right") - 1
    for e in np.unique(e_of):
        sel = pairs[e_of == e]
        o1 = prep_rows(sel if a_rows is None else a_rows[sel])
        wc, ws = w_rows(e, np.concatenate([cols, I + cols]))
        y, b = linear_ref(o1["bb_codes"], o1["bb_scales"], o1["res_codes"], o1["res_scales"], wc, ws)
        assert_h_close(h_np[np.ix_(sel, cols)], y[:, :nc], b[:, :nc], y[:, nc:], b[:, nc:])


def _check(sq, p1, w_gu, seg, a_rows, P, I, n, m, pairs):
    import torch
    seg_g = i32_to_gpu(seg)
    rows_g = None if a_rows is None else i32_to_gpu(a_rows)
    y = sq.linear_grouped(p1, w_gu, seg_g, rows_g)
    h_ref = sq.silu_mul(y)
    p2_ref = sq.prepare(h_ref, None, n, m)
    hp, h = sq.linear_grouped_silu_prepare(p1, w_gu, seg_g, rows_g, n, m, with_h=True)
    torch.cuda.synchronize()
    assert h.shape == (P, I)
    assert np.array_equal(to_np(h), to_np(h_ref)), "fused h differs from linear_grouped -> silu_mul"
    for f in FIELDS:
        assert np.array_equal(to_np(getattr(hp, f)), to_np(getattr(p2_ref, f))), f"fused {f} differs"
    # prepared output only (no mask), into a preallocated Prepared
    hp2, h2 = sq.linear_grouped_silu_prepare(p1, w_gu, seg_g, rows_g, n, m, with_mask=False)
    assert h2 is None and hp2.mask is None
    for f in FIELDS[:4]:
        assert np.array_equal(to_np(getattr(hp2, f)), to_np(getattr(p2_ref, f)))
    hp3, _ = sq.linear_grouped_silu_prepare(p1, w_gu, seg_g, rows_g, n, m, out=hp2)
    assert hp3 is hp2
    # the oracle on sampled pairs
    h_np = to_np(h)
    assert_prepare_equal(hp, prepare_ref(h_np[pairs], None, n, m), rows=pairs)
    assert_bf16_close(h_np[pairs], silu_mul_ref(to_np(y)[pairs], I))
    return h_np


@pytest.mark.parametrize("use_rows,n,m", [(True, 2, 4), (False, 8, 16), (True, 8, 16)])
def test_grouped_fused_small_with_empty_and_single_row_experts(sq, use_rows, n, m):
    print(f"grouped fused small a_rows={use_rows} {n}:{m}", flush=True)
    rng = np.random.default_rng(31 + n)
    tokens, E, K, I = 300, 7, 256, 256
    x = bf16_round((rng.standard_normal((tokens, K)) * 3).astype(np.float32))
    p = prepare_ref(x, None, 2, 4)
    wq = [quantize_weight_ref(bf16_round((rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32)))
          for _ in range(E)]
    wc, ws = np.stack([c for c, _ in wq]), np.stack([s for _, s in wq])
    if use_rows:
        a_rows, _, _, _ = moe_routing(rng, tokens, E, 2)
        P = len(a_rows)
        seg = np.array([0, 150, 300, 300, 420, 421, 500, P], np.int32)  # expert 2 empty, expert 4 one row
    else:
        a_rows = None
        P = tokens
        seg = np.array([0, 1, 1, 130, 131, 260, 299, P], np.int32)
    pairs = np.unique(np.concatenate([seg[:-1][seg[:-1] < P], [P - 1], rng.choice(P, 30, replace=False)]))
    h_np = _check(sq, oracle_prepared(p), w_to_gpu(wc, ws), seg, a_rows, P, I, n, m, pairs)
    _check_h_oracle(h_np, pairs, seg, a_rows, I, lambda src: {f: p[f][src] for f in p},
                    lambda e, r: (wc[e][r], ws[e][r]), seed=n)


def test_grouped_fused_qwen3_full_size(sq):
    print("grouped fused gate|up workload qwen3 moe 32768 pairs x 2048 -> 2 x 768", flush=True)
    wl = workload_qwen3_moe()
    E, I, H = wl["experts"], wl["inter"], wl["hidden"]
    a_rows, seg = wl["a_rows"], wl["seg_offsets"]
    P = len(a_rows)
    w_gu = sq.quantize_mxfp4(bf16_to_gpu(wl["w_gu"].reshape(E * 2 * I, H)).view(E, 2 * I, H))
    p1 = sq.prepare(bf16_to_gpu(wl["x"]), None, 2, 4)
    rng = np.random.default_rng(13)
    pairs = np.unique(np.concatenate([seg[:-1][seg[:-1] < P][::9], rng.choice(P, 40, replace=False), [P - 1]]))
    h_np = _check(sq, p1, w_gu, seg, a_rows, P, I, 2, 4, pairs)
    _check_h_oracle(h_np, pairs, seg, a_rows, I, lambda src: prepare_ref(wl["x"][src], None, 2, 4),
                    lambda e, r: quantize_weight_ref(wl["w_gu"][e][r]), seed=5)
