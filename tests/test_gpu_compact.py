"""GPU parity of the compressed sparse backbone (sharq_compress_backbone,
sharq_expand_backbone) against the oracle: the compressed codes and the rank
fields bit for bit, and the lossless round trip back to the dense stage-major
codes (padding blocks zero) and the mask, for 2:4 and 8:16, ragged row counts,
a K with a half stage, and the down-projection input at full size."""

import numpy as np
import pytest

from oracle import compress_backbone_ref, expand_backbone_ref, meta_row_bytes, prepare_ref
from synth import bf16_round
from gpu_util import bf16_to_gpu, codes_row_major, codes_stage_major, to_np, u8_to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import activation_sparsity_fp4_amd as sq
    return sq


def _x(T, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * rng.lognormal(0, 1, (T, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 40
    x[min(2, T - 1), :] = 0  # a zero row keeps the lowest positions of every group
    return bf16_round(x)


@pytest.mark.parametrize("T,K,n,m", [(37, 256, 2, 4), (37, 256, 8, 16), (300, 1088, 2, 4), (129, 1088, 8, 16),
                                     (1, 64, 2, 4), (64, 4096, 8, 16)])
def test_compress_and_expand_match_oracle(sq, T, K, n, m):
    print(f"compact backbone T={T} K={K} {n}:{m}", flush=True)
    x = _x(T, K, T + K + n)
    prep = sq.prepare(bf16_to_gpu(x), None, n, m)
    cb = sq.compress_backbone(prep, n, m)
    want = prepare_ref(x, None, n, m)
    wc, wm = compress_backbone_ref(want["bb_codes"], want["mask"], n, m)
    assert cb.meta.shape[1] == meta_row_bytes(K, n, m)
    assert np.array_equal(to_np(cb.codes), wc), "compressed codes differ from the oracle"
    assert np.array_equal(to_np(cb.meta), wm), "rank fields differ from the oracle"
    bb, mask = sq.expand_backbone(cb)
    assert np.array_equal(to_np(bb), to_np(prep.bb_codes)), "round trip: codes (padding blocks included)"
    assert np.array_equal(to_np(mask), to_np(prep.mask)), "round trip: mask"
    # expanding the oracle's compressed form gives the oracle's expansion
    cb2 = sq.CompactBackbone(u8_to_gpu(wc), u8_to_gpu(wm), n, m, K)
    bb2, mask2 = sq.expand_backbone(cb2)
    ob, om = expand_backbone_ref(wc, wm, K, n, m)
    assert np.array_equal(codes_row_major(to_np(bb2), K // 2), ob)
    assert np.array_equal(to_np(mask2), om)
    # no mask requested
    bb3, m3 = sq.expand_backbone(cb2, with_mask=False)
    assert m3 is None and np.array_equal(to_np(bb3), to_np(bb2))


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16)])
def test_compact_down_input_full_size(sq, n, m):
    # the down projection's input, 2048 x 14336: round trip in full, the oracle on sampled rows
    print(f"compact backbone 2048x14336 {n}:{m}", flush=True)
    T, K = 2048, 14336
    rng = np.random.default_rng(9)
    g = rng.standard_normal((T, K)).astype(np.float32)
    u = rng.standard_normal((T, K)).astype(np.float32)
    x = bf16_round(g / (1 + np.exp(-g)) * u)
    prep = sq.prepare(bf16_to_gpu(x), None, n, m)
    cb = sq.compress_backbone(prep, n, m)
    bb, mask = sq.expand_backbone(cb)
    assert np.array_equal(to_np(bb), to_np(prep.bb_codes)) and np.array_equal(to_np(mask), to_np(prep.mask))
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 40, replace=False)]))
    want = prepare_ref(x[rows], None, n, m)
    wc, wm = compress_backbone_ref(want["bb_codes"], want["mask"], n, m)
    assert np.array_equal(to_np(cb.codes)[rows], wc) and np.array_equal(to_np(cb.meta)[rows], wm)
