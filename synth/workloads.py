"""Seeded workload generators (numpy PCG64; one SeedSequence per workload).

Activations follow the outlier model used for every workload: standard normal
entries, a seeded set of outlier channels multiplied by a constant factor, and a
per-token lognormal(0, 0.5) scale. Weights are N(0, 0.02). Every array is drawn
in float32 and rounded once to bf16 (round to nearest even) and returned as
uint16 bit patterns.

Workloads (tokens x features):
  linear_128x4096       X [128 x 4096] 2:4, W [4096 x 4096]
  llama8b_mlp           X [2048 x 4096] 2:4 + gamma ~ U(0.5, 1.5); gate|up W
                        [28672 x 4096] (gate rows first); down W [4096 x 14336]
  down_silu_8of16       X = SiLU(g) * u [2048 x 14336], 1% channels x30; W [4096 x 14336]
  llama70b_decode       X [T x 8192], T in {1, 8, 32, 64}; gate|up W [57344 x 8192];
                        down W [8192 x 28672]
  qwen3_moe             4096 tokens x 2048; 128 experts, top-8 routing from
                        softmax(N(0,1) logits); per-expert gate|up W [1536 x 2048]
                        and down W [2048 x 768]
Sizes can be shrunk (same distributions) for fast tests.
"""

from __future__ import annotations

import hashlib

import numpy as np

__all__ = [
    "SEEDS",
    "bf16_round",
    "bf16_to_f32",
    "outlier_activation",
    "normal_weight",
    "workload_linear",
    "workload_llama8b_mlp",
    "workload_down_silu",
    "workload_llama70b_decode",
    "workload_qwen3_moe",
    "moe_routing",
    "moe_combine_index",
    "array_digest",
    "adversarial_rows",
]

SEEDS = {
    "linear_128x4096": 1001,
    "llama8b_mlp": 1002,
    "down_silu_8of16": 1003,
    "llama70b_decode": 1004,
    "qwen3_moe": 1005,
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    rounded = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, count: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(count)]


def outlier_activation(rng_x, rng_ch, rng_tok, T: int, K: int, frac: float = 0.005,
                       factor: float = 50.0, token_sigma: float = 0.5) -> np.ndarray:
    """float32 [T x K]: N(0,1) * (factor on round(frac*K) seeded channels) * lognormal(0, sigma) per token."""
    z = rng_x.standard_normal((T, K), dtype=np.float32)
    n_out = int(round(frac * K))
    ch = np.sort(rng_ch.choice(K, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    c = np.ones(K, dtype=np.float32)
    c[ch] = np.float32(factor)
    s = rng_tok.lognormal(0.0, token_sigma, size=(T, 1)).astype(np.float32)
    return z * c[None, :] * s


def normal_weight(rng, O: int, K: int, sigma: float = 0.02, chunk_rows: int = 4096) -> np.ndarray:
    """bf16 bits [O x K] with N(0, sigma) entries, generated in row chunks to bound memory."""
    out = np.empty((O, K), dtype=np.uint16)
    for r in range(0, O, chunk_rows):
        rr = min(chunk_rows, O - r)
        w = rng.standard_normal((rr, K), dtype=np.float32) * np.float32(sigma)
        out[r:r + rr] = bf16_round(w)
    return out


def workload_linear(seed: int = SEEDS["linear_128x4096"], T: int = 128, K: int = 4096, O: int = 4096):
    """Single linear layer, 2:4: X bf16 [T x K] with the outlier model, W [O x K]."""
    rx, rc, rt, rw = _streams(seed, 4)
    x = bf16_round(outlier_activation(rx, rc, rt, T, K))
    w = normal_weight(rw, O, K)
    return {"x": x, "w": w, "n": 2, "m": 4}


def workload_llama8b_mlp(seed: int = SEEDS["llama8b_mlp"], T: int = 2048, hidden: int = 4096,
                         inter: int = 14336, with_weights: bool = True):
    """Llama-3.1-8B-shaped MLP block, 2:4, gamma absorbed in the first prepare."""
    rx, rc, rt, rg, rw1, rw2 = _streams(seed, 6)
    x = bf16_round(outlier_activation(rx, rc, rt, T, hidden))
    gamma = bf16_round(rg.uniform(0.5, 1.5, size=hidden).astype(np.float32))
    out = {"x": x, "gamma": gamma, "n": 2, "m": 4, "hidden": hidden, "inter": inter}
    if with_weights:
        out["w_gu"] = normal_weight(rw1, 2 * inter, hidden)  # gate rows [0, I), up rows [I, 2I)
        out["w_down"] = normal_weight(rw2, hidden, inter)
    return out


def workload_down_silu(seed: int = SEEDS["down_silu_8of16"], T: int = 2048, K: int = 14336,
                       O: int = 4096, with_weights: bool = True):
    """down_proj input X = SiLU(g) * u, g, u ~ N(0,1), 1% outlier channels x30; run 8:16 and 2:4."""
    rg, ru, rc, rw = _streams(seed, 4)
    g = rg.standard_normal((T, K), dtype=np.float32)
    u = ru.standard_normal((T, K), dtype=np.float32)
    h = g / (np.float32(1) + np.exp(-g)) * u
    n_out = int(round(0.01 * K))
    ch = np.sort(rc.choice(K, size=n_out, replace=False))
    h[:, ch] *= np.float32(30.0)
    out = {"x": bf16_round(h), "n": 8, "m": 16}
    if with_weights:
        out["w"] = normal_weight(rw, O, K)
    return out


def workload_llama70b_decode(T: int, seed: int = SEEDS["llama70b_decode"], hidden: int = 8192,
                             inter: int = 28672, with_weights: bool = True):
    """Llama-3.1-70B-shaped decode GEMMs, 2:4, T tokens (1, 8, 32 or 64)."""
    rx, rc, rt, rw1, rw2 = _streams(seed, 5)
    x = bf16_round(outlier_activation(rx, rc, rt, T, hidden))
    out = {"x": x, "n": 2, "m": 4, "hidden": hidden, "inter": inter}
    if with_weights:
        out["w_gu"] = normal_weight(rw1, 2 * inter, hidden)
        out["w_down"] = normal_weight(rw2, hidden, inter)
    return out


def moe_routing(rng, tokens: int, experts: int, top_k: int):
    """Top-k routing from softmax(N(0,1) logits); ties go to the lower expert index.

    Returns (a_rows [P] int32 token of each sorted pair, seg_offsets [E+1] int32,
    expert_of_pair [P] int32, weight_of_pair [P] float32) with pairs sorted stably
    by expert (token order preserved inside an expert)."""
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :top_k]  # [tokens, k]
    wts = np.take_along_axis(p, order, axis=1)
    tok = np.repeat(np.arange(tokens), top_k)
    exp = order.reshape(-1)
    srt = np.argsort(exp, kind="stable")
    a_rows = tok[srt].astype(np.int32)
    e_sorted = exp[srt].astype(np.int32)
    counts = np.bincount(e_sorted, minlength=experts)
    seg = np.zeros(experts + 1, dtype=np.int32)
    seg[1:] = np.cumsum(counts)
    return a_rows, seg, e_sorted, wts.reshape(-1)[srt].astype(np.float32)


def moe_combine_index(a_rows: np.ndarray, weight_of_pair: np.ndarray, tokens: int, top_k: int):
    """Token-major view of a routing (indexing only): pair_index [tokens, top_k]
    int32 lists the sorted pairs of each token in sorted-pair order (-1 for an
    empty slot), weights [tokens, top_k] float32 their routing weights (0 for an
    empty slot)."""
    a_rows = np.asarray(a_rows)
    order = np.argsort(a_rows, kind="stable")  # pairs grouped by token, sorted-pair order inside
    counts = np.bincount(a_rows, minlength=tokens)
    if counts.max(initial=0) > top_k:
        raise ValueError("a token has more pairs than top_k")
    pair_index = np.full((tokens, top_k), -1, dtype=np.int32)
    weights = np.zeros((tokens, top_k), dtype=np.float32)
    start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    slot = np.arange(len(order)) - np.repeat(start, counts)
    tok = a_rows[order]
    pair_index[tok, slot] = order.astype(np.int32)
    weights[tok, slot] = np.asarray(weight_of_pair, dtype=np.float32)[order]
    return pair_index, weights


def workload_qwen3_moe(seed: int = SEEDS["qwen3_moe"], tokens: int = 4096, hidden: int = 2048,
                       experts: int = 128, inter: int = 768, top_k: int = 8, with_weights: bool = True):
    """Qwen3-30B-A3B-shaped MoE expert layer, 2:4, grouped over token-sorted expert segments."""
    rx, rc, rt, rr, rw1, rw2 = _streams(seed, 6)
    x = bf16_round(outlier_activation(rx, rc, rt, tokens, hidden))
    a_rows, seg, e_of_pair, w_of_pair = moe_routing(rr, tokens, experts, top_k)
    out = {"x": x, "n": 2, "m": 4, "a_rows": a_rows, "seg_offsets": seg,
           "expert_of_pair": e_of_pair, "weight_of_pair": w_of_pair,
           "hidden": hidden, "inter": inter, "experts": experts}
    if with_weights:
        w_gu = np.empty((experts, 2 * inter, hidden), dtype=np.uint16)
        w_dn = np.empty((experts, hidden, inter), dtype=np.uint16)
        for e in range(experts):
            w_gu[e] = normal_weight(rw1, 2 * inter, hidden)
        for e in range(experts):
            w_dn[e] = normal_weight(rw2, hidden, inter)
        out["w_gu"] = w_gu
        out["w_down"] = w_dn
    return out


def array_digest(a: np.ndarray) -> str:
    """Short SHA-256 of an array's bytes (recorded next to bench results)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def adversarial_rows(K: int, seed: int = 0) -> np.ndarray:
    """float32 rows [10 x K] that stress edge cases: zeros, alternating +-0, constant
    rows (all ties), bf16 subnormals, small-alphabet ties, mixed normal/subnormal,
    huge outliers, values near the fp32 range, powers of two over the whole bf16
    exponent range, and values that land between 6 and 8 after block scaling."""
    rng = np.random.default_rng(seed)
    rows = [
        np.zeros(K),
        np.where(np.arange(K) % 2, -0.0, 0.0),
        np.full(K, 1.5),
        np.full(K, -2.0 ** -130),
        rng.choice([1.0, -1.0, 2.0, 0.0], size=K),
        rng.standard_normal(K) * 2.0 ** -128,
    ]
    big = rng.standard_normal(K)
    big[::13] *= 1e30
    rows.append(big)
    rows.append(rng.standard_normal(K) * 1e37)
    rows.append(np.ldexp(1.0, rng.integers(-133, 127, K)) * rng.choice([-1, 1], K))
    sat = rng.standard_normal(K)
    sat[::32] = 7.0
    rows.append(sat)
    return np.array(rows, dtype=np.float32)
