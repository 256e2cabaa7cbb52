"""Oracle of the compressed sparse backbone (test infrastructure only: the same
rules as ``sharq_ref`` apply -- only tests, smoke() and the bench's CPU
baseline may call it, and it shares nothing with the HIP library).

What the pages fix: the SharQ page (Abstract) names a "sparse input
compression" inside the fused prepare without defining it; the 8:16 page
(abstract) states the storage cost of an N:M mask as 0.75 bits per element for
2:4 and 0.875 for 8:16, which is ceil(log2 C(M, N)) bits per group of M:
C(4, 2) = 6 patterns in 3 bits, C(16, 8) = 12870 patterns in 14 bits.

Reading taken where they are silent:
* the compressed backbone of a row keeps, for every group of M, the N codes at
  the kept positions in index order (N/M of the dense nibbles), and one
  metadata field per group holding the rank of the kept position set;
* the rank is the combinatorial number system in colexicographic order: for
  kept positions c_1 < ... < c_N (0-based inside the group),
  rank = C(c_1, 1) + C(c_2, 2) + ... + C(c_N, N), a bijection onto
  [0, C(M, N));
* each row's fields are a bit stream, group g at bits [g b, g b + b) with
  b = ceil(log2 C(M, N)), least significant bit first, padded to whole bytes;
* compressed codes are packed two per byte, the earlier one in the low nibble
  (as the dense codes).
Block scales are unchanged (the backbone's 32-blocks keep their E8M0 bytes).
"""

from __future__ import annotations

import math

import numpy as np

from .sharq_ref import pack_mask, pack_nibbles, unpack_mask, unpack_nibbles

__all__ = ["meta_bits", "meta_row_bytes", "subset_rank", "subset_unrank", "compress_backbone_ref",
           "expand_backbone_ref"]


def meta_bits(n: int, m: int) -> int:
    """Bits of one group's field: ceil(log2 C(m, n))."""
    return max(1, math.ceil(math.log2(math.comb(m, n))))


def meta_row_bytes(K: int, n: int, m: int) -> int:
    """Bytes of one row's metadata stream (K / m fields, padded to bytes)."""
    if K % m:
        raise ValueError("K must be a multiple of m")
    return (K // m * meta_bits(n, m) + 7) // 8


def subset_rank(positions, n: int) -> int:
    """Colex rank of a set of n positions: sum over the sorted positions c_i
    (i = 1..n) of C(c_i, i)."""
    c = sorted(positions)
    if len(c) != n or len(set(c)) != n:
        raise ValueError("need n distinct positions")
    return sum(math.comb(ci, i + 1) for i, ci in enumerate(c))


def subset_unrank(rank: int, m: int, n: int) -> tuple:
    """Inverse of subset_rank: the largest c_n with C(c_n, n) <= rank, then the
    same for n - 1 on the remainder, and so on."""
    if not 0 <= rank < math.comb(m, n):
        raise ValueError("rank out of range")
    out = []
    r = rank
    top = m
    for i in range(n, 0, -1):
        c = i - 1
        while c + 1 < top and math.comb(c + 1, i) <= r:
            c += 1
        r -= math.comb(c, i)
        out.append(c)
        top = c
    if r != 0:
        raise AssertionError("unrank did not consume the rank")
    return tuple(sorted(out))


def _comb_table(m: int, n: int) -> np.ndarray:
    """comb[p, i] = C(p, i) for p < m, i <= n (int64)."""
    return np.array([[math.comb(p, i) for i in range(n + 1)] for p in range(m)], dtype=np.int64)


def compress_backbone_ref(bb_codes: np.ndarray, mask: np.ndarray, n: int, m: int):
    """Compress a backbone: bb_codes u8 [T, K/2] (dense-masked, packed nibbles)
    and mask u8 [T, K/8] -> (codes u8 [T, K n / (2 m)], meta u8 [T, meta_row_bytes]).

    Dense codes at dropped positions must be 0 (they carry nothing)."""
    codes = unpack_nibbles(bb_codes)
    keep = unpack_mask(mask)
    T, K = codes.shape
    if keep.shape != (T, K) or K % m:
        raise ValueError("shapes")
    groups = keep.reshape(T, K // m, m)
    if not np.all(groups.sum(axis=-1) == n):
        raise ValueError("every group must keep exactly n positions")
    if np.any(codes[~keep] != 0):
        raise ValueError("dropped positions must hold code 0")
    # kept codes in index order: a stable selection of the kept positions
    kept = codes.reshape(T, K // m, m)[groups].reshape(T, K // m * n)
    out_codes = pack_nibbles(kept)
    # rank of each group's kept set: sum over kept p of C(p, number of kept positions up to p)
    comb = _comb_table(m, n)
    ordinal = np.cumsum(groups, axis=-1)  # i for the i-th kept position (1-based)
    pos = np.broadcast_to(np.arange(m), groups.shape)
    contrib = np.where(groups, comb[pos, np.minimum(ordinal, n)], 0)
    rank = contrib.sum(axis=-1).astype(np.int64)  # [T, K/m]
    b = meta_bits(n, m)
    bits = ((rank[:, :, None] >> np.arange(b)[None, None, :]) & 1).astype(np.uint8).reshape(T, -1)
    nbytes = meta_row_bytes(K, n, m)
    padded = np.zeros((T, nbytes * 8), dtype=np.uint8)
    padded[:, :bits.shape[1]] = bits
    meta = np.packbits(padded.reshape(T, nbytes, 8), axis=-1, bitorder="little").reshape(T, nbytes)
    return out_codes, meta


def expand_backbone_ref(codes: np.ndarray, meta: np.ndarray, K: int, n: int, m: int):
    """Inverse of compress_backbone_ref: -> (bb_codes u8 [T, K/2], mask u8 [T, K/8])."""
    codes = np.asarray(codes, dtype=np.uint8)
    meta = np.asarray(meta, dtype=np.uint8)
    T = codes.shape[0]
    b = meta_bits(n, m)
    G = K // m
    bits = np.unpackbits(meta, axis=-1, bitorder="little")[:, :G * b].reshape(T, G, b).astype(np.int64)
    rank = (bits << np.arange(b)[None, None, :]).sum(axis=-1)
    if np.any(rank >= math.comb(m, n)):
        raise ValueError("metadata field out of range")
    keep = np.zeros((T, G, m), dtype=bool)
    for r in np.unique(rank):
        keep[rank == r] = np.isin(np.arange(m), subset_unrank(int(r), m, n))
    kept = unpack_nibbles(codes).reshape(T, G, n)
    dense = np.zeros((T, G, m), dtype=np.uint8)
    dense[keep] = kept.reshape(-1)
    return pack_nibbles(dense.reshape(T, K)), pack_mask(keep.reshape(T, K))
