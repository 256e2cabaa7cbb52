"""Pins for the oracle's N:M selection (CPU only).

The oracle sorts by magnitude; these tests check it against a different
formulation -- exhaustive enumeration of every N-of-M subset, choosing the one
with the largest exact sum of |x| and, among equal sums, the lexicographically
smallest index tuple -- and against the storage and pruning-rate figures the
pages print.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import select_nm, pack_mask, unpack_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_keep(group, n):
    """Subset of size n maximising sum |x| exactly; ties -> lexicographically smallest tuple."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(group)), n):  # lexicographic order
        s = sum(abs(Fraction(float(group[i]))) for i in sub)
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    keep = np.zeros(len(group), dtype=bool)
    keep[list(best)] = True
    return keep


def test_2of4_exhaustive_small_alphabet():
    # every 2:4 group over {0, -0, +-1, +-2, +-3}: 9**4 = 6561 groups, full of ties
    alphabet = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0, 0.5]
    groups = np.array(list(itertools.product(alphabet, repeat=4)), dtype=np.float32)
    got = select_nm(groups.reshape(-1, 4), 2, 4)
    for g, k in zip(groups, got):
        assert np.array_equal(k, brute_force_keep(g, 2)), g


def _subset_matrix(m, n):
    subs = list(itertools.combinations(range(m), n))
    mat = np.zeros((len(subs), m), dtype=np.int64)
    for i, s in enumerate(subs):
        mat[i, list(s)] = 1
    return mat


@pytest.mark.parametrize("n,m", [(8, 16), (2, 4), (1, 4), (4, 8)])
def test_nm_bruteforce_random_with_ties(n, m):
    rng = np.random.default_rng(7)
    mat = _subset_matrix(m, n)  # rows in lexicographic order of combinations
    # small integer magnitudes force many ties; random signs
    for trial in range(200):
        vals = rng.integers(0, 4 if trial % 2 else 50, size=m)
        signs = rng.choice([-1.0, 1.0], size=m)
        g = (vals * signs).astype(np.float32)
        sums = mat @ np.abs(vals)  # exact integers
        best = int(np.flatnonzero(sums == sums.max())[0])  # first = lexicographically smallest
        want = mat[best].astype(bool)
        got = select_nm(g[None, :], n, m)[0]
        assert np.array_equal(got, want), (g, got, want)


def test_all_equal_and_zero_groups_pick_lowest_indices():
    for n, m in [(2, 4), (8, 16)]:
        for v in [0.0, -0.0, 1.5, -7.0]:
            g = np.full((1, m), v, dtype=np.float32)
            keep = select_nm(g, n, m)[0]
            assert np.array_equal(keep, np.arange(m) < n)
        # +0 and -0 tie; opposite signs of equal magnitude tie
        g = np.array([[-0.0, 0.0, -0.0, 0.0]], dtype=np.float32)
        assert np.array_equal(select_nm(g, 2, 4)[0], [True, True, False, False])
        g = np.array([[-2.0, 1.0, 2.0, -1.0]], dtype=np.float32)
        assert np.array_equal(select_nm(g, 2, 4)[0], [True, False, True, False])


def test_mask_invariants_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((37, 256)) * rng.lognormal(0, 2, (37, 256))).astype(np.float32)
    x[:, ::7] = 0
    for n, m in [(2, 4), (8, 16)]:
        keep = select_nm(x, n, m)
        g = keep.reshape(37, -1, m)
        assert np.all(g.sum(-1) == n)
        a = np.abs(x).reshape(37, -1, m)
        kept_min = np.where(g, a, np.inf).min(-1)
        drop_max = np.where(~g, a, -np.inf).max(-1)
        assert np.all(kept_min >= drop_max)
        # at equal magnitude a kept entry never sits after a dropped one
        for t in range(0, 37, 5):
            for j in range(g.shape[1]):
                for i1 in range(m):
                    for i2 in range(i1 + 1, m):
                        if a[t, j, i1] == a[t, j, i2] and g[t, j, i2]:
                            assert g[t, j, i1]


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_pruning_rate_matches_page():
    # Module 6, formula 1 of the challenge page: R = N_pruned / N_total; 2:4 -> 50.00%
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    for n, m, pct in _read_golden("pruning_rate.txt"):
        keep = select_nm(x, int(n), int(m))
        rate = 100.0 * (~keep).sum() / keep.size
        assert rate == float(pct)


def test_mask_pattern_count_matches_page_storage_bits():
    # The 8:16 page prints 0.875 vs 0.75 bits/element for the mask. Check that the
    # oracle's selection can produce exactly C(m, n) distinct group masks and that
    # ceil(log2 C(m, n)) / m reproduces the printed figures.
    for n, m, bits in _read_golden("nm_mask_bits.txt"):
        n, m, bits = int(n), int(m), float(bits)
        subs = list(itertools.combinations(range(m), n))
        xs = np.ones((len(subs), m), dtype=np.float32)
        for i, s in enumerate(subs):
            xs[i, list(s)] = 5.0
        keep = select_nm(xs, n, m)
        patterns = {tuple(k) for k in keep}
        assert len(patterns) == math.comb(m, n)
        assert math.ceil(math.log2(len(patterns))) / m == bits


def test_mask_packing_bit_order():
    keep = np.zeros((2, 16), dtype=bool)
    keep[0, [0, 3, 9, 15]] = True
    keep[1, [1, 2]] = True
    packed = pack_mask(keep)
    assert packed.tolist() == [[0b00001001, 0b10000010], [0b00000110, 0]]
    assert np.array_equal(unpack_mask(packed), keep)
