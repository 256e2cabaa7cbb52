"""Pins of the compressed-backbone oracle (the sparse input compression named
on the SharQ page, Abstract): the metadata field is the colex rank of the kept
set, checked against its definition by brute-force enumeration of every
subset; its size against the bits per element printed on the 8:16 page
(abstract, tests/golden/nm_mask_bits.txt); a hand-worked row; and lossless
round trips of real prepare outputs."""

import itertools
import math
import os

import numpy as np
import pytest

from oracle import (compress_backbone_ref, expand_backbone_ref, meta_bits, meta_row_bytes, pack_mask, pack_nibbles,
                    prepare_ref, subset_rank, subset_unrank, unpack_mask, unpack_nibbles)
from synth import bf16_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nm_mask_bits.txt")


@pytest.mark.parametrize("m,n", [(4, 2), (16, 8), (8, 3), (6, 1), (5, 5)])
def test_rank_is_the_colex_index(m, n):
    # every n-subset of range(m), ordered colexicographically (by the largest position, then the next ...):
    # the rank is the index in that list, and unrank inverts it
    subsets = sorted(itertools.combinations(range(m), n), key=lambda c: tuple(reversed(c)))
    assert len(subsets) == math.comb(m, n)
    for idx, c in enumerate(subsets):
        assert subset_rank(c, n) == idx
        assert subset_unrank(idx, m, n) == c


def test_bits_per_element_match_the_page():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 2
    for n, m, bits in rows:
        n, m, bits = int(n), int(m), float(bits)
        assert meta_bits(n, m) == math.ceil(math.log2(math.comb(m, n)))
        for K in (64, 4096, 14336):
            assert meta_row_bytes(K, n, m) * 8 / K == bits


def test_hand_worked_2of4_row():
    # codes of 8 positions; groups keep {0, 2} (rank C(0,1) + C(2,2) = 1) and {1, 3} (rank C(1,1) + C(3,2) = 4)
    codes = np.array([[3, 0, 5, 0, 0, 9, 0, 0xA]], np.uint8)
    keep = np.array([[1, 0, 1, 0, 0, 1, 0, 1]], bool)
    cc, meta = compress_backbone_ref(pack_nibbles(codes), pack_mask(keep), 2, 4)
    assert cc.tolist() == [[0x53, 0xA9]]            # kept codes 3, 5, 9, A in index order, low nibble first
    assert meta.tolist() == [[0b00100001]]          # fields 1 = 001b and 4 = 100b, least significant bit first
    bb, mk = expand_backbone_ref(cc, meta, 8, 2, 4)
    assert np.array_equal(unpack_nibbles(bb), codes) and np.array_equal(unpack_mask(mk), keep)


@pytest.mark.parametrize("n,m,K", [(2, 4, 256), (8, 16, 256), (2, 4, 4096), (8, 16, 1024)])
def test_round_trip_of_prepare_outputs(n, m, K):
    rng = np.random.default_rng(K + n)
    x = bf16_round((rng.standard_normal((24, K)) * rng.lognormal(0, 1, (24, 1))).astype(np.float32))
    x[3, :] = 0  # an all-zero row: every group keeps its lowest positions
    p = prepare_ref(x, None, n, m)
    cc, meta = compress_backbone_ref(p["bb_codes"], p["mask"], n, m)
    assert cc.shape == (24, K * n // m // 2) and meta.shape == (24, meta_row_bytes(K, n, m))
    bb, mk = expand_backbone_ref(cc, meta, K, n, m)
    assert np.array_equal(bb, p["bb_codes"]) and np.array_equal(mk, p["mask"])
    # the compressed codes are the kept codes, gathered one by one
    dense, keep = unpack_nibbles(p["bb_codes"]), unpack_mask(p["mask"])
    for t in (0, 3, 23):
        assert unpack_nibbles(cc)[t].tolist() == [int(dense[t, k]) for k in range(K) if keep[t, k]]


def test_expand_rejects_fields_out_of_range():
    meta = np.full((1, meta_row_bytes(64, 8, 16)), 0xFF, np.uint8)  # fields 16383 >= C(16, 8) = 12870
    with pytest.raises(ValueError):
        expand_backbone_ref(np.zeros((1, 16), np.uint8), meta, 64, 8, 16)
