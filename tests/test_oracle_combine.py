"""Pins of the MoE weighted-combine oracle: a hand-worked two-token case, the
single-slot unit-weight case reducing to a row gather, linearity in y and in
the weights, and agreement with a per-element Python loop on a routed case."""

import numpy as np

from oracle import moe_combine_ref
from synth import moe_combine_index, moe_routing


def test_hand_worked():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    idx = np.array([[0, 2], [1, -1]], np.int32)
    w = np.array([[0.5, 0.25], [2.0, 7.0]], np.float32)
    out, bound = moe_combine_ref(y, idx, w)
    assert out.tolist() == [[25.5, 51.0], [20.0, 40.0]]
    assert bound.tolist() == [[25.5, 51.0], [20.0, 40.0]]


def test_single_slot_is_a_gather_and_linearity():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((50, 16))
    idx = rng.permutation(50)[:20].reshape(20, 1).astype(np.int32)
    out, _ = moe_combine_ref(y, idx, np.ones((20, 1), np.float32))
    assert np.array_equal(out, y[idx[:, 0]])
    idx2 = rng.integers(-1, 50, (20, 4)).astype(np.int32)
    w = rng.uniform(0, 1, (20, 4)).astype(np.float32)
    a, _ = moe_combine_ref(y, idx2, w)
    b, _ = moe_combine_ref(2 * y, idx2, w)
    c, _ = moe_combine_ref(y, idx2, 2 * w)
    assert np.array_equal(b, 2 * a) and np.array_equal(c, 2 * a)


def test_routed_case_against_a_loop():
    rng = np.random.default_rng(2)
    T, E, k, H = 40, 8, 3, 5
    a_rows, seg, _, w_pair = moe_routing(rng, T, E, k)
    idx, w = moe_combine_index(a_rows, w_pair, T, k)
    assert (idx >= 0).all() and sorted(idx.reshape(-1).tolist()) == list(range(T * k))
    assert np.array_equal(a_rows[idx], np.repeat(np.arange(T), k).reshape(T, k))
    y = rng.standard_normal((T * k, H))
    out, _ = moe_combine_ref(y, idx, w)
    for t in range(T):
        for h in range(H):
            want = 0.0
            for j in range(k):
                want += float(w[t, j]) * y[idx[t, j], h]
            assert abs(out[t, h] - want) <= 1e-12 * (1 + abs(want))
