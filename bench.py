#!/usr/bin/env python3
"""Benchmark of the SharQ linear hot path on one MI355X.

Headline workload: a Llama-3.1-8B-shaped MLP block at 2048-token prefill, 2:4,
MXFP4, the RMSNorm (per-row 1/rms and gamma) absorbed in the first prepare:
    prepare(rmsnorm(x)) -> fused [two-path GEMM gate|up [28672 x 4096] ->
    silu(gate) * up -> prepare(h)] -> two-path GEMM down [4096 x 14336]
One step = one pass of that chain over 2048 tokens. Inputs are seeded synthetic
data resident in HBM before the timed region; weights are quantised once on
the GPU (not timed).

Timed region: K replays of the step captured once as a HIP graph (kernel
nodes only; inside it the kernels run back to back), HIP events recorded on
the launch stream before and after them; `value` is tokens over the
wall-clock time of the K steps. Before it, W warm-up steps and half a second
of untimed replays: the GPU boosts its clocks for the first milliseconds of a
load and then settles to its sustained (power-limited) clock, which is what
the timed region measures. Stage (kernel) times come from a graph of back-to-back
launches of each stage alone, HIP events around its replays. The same step
launched eagerly (HIP events between the stages) is reported beside it.

Prints ONE JSON line: tokens/s, the per-stage breakdown, the roofline of the
dominant kernel, a `configs` object with the other workloads (single linear
128x4096, down_proj 2048x14336 8:16 and 2:4, Llama-3.1-70B decode at T = 1, 8,
32, 64 with three rotated weight copies, Qwen3-30B-A3B MoE layer) and the CPU
oracle timed in a child process on a bounded sample of the headline workload.
Other workloads as the headline: --workload NAME.
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 scaled MFMA
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 MFMA (the NVFP4 GEMM widens its codes to fp16)

WORKLOADS = ["llama8b_mlp", "linear_128x4096", "down_8of16", "down_2of4", "llama70b_decode_T1",
             "llama70b_decode_T8", "llama70b_decode_T32", "llama70b_decode_T64", "qwen3_moe", "compact_2of4",
             "compact_8of16", "nvfp4_down_8of16", "nvfp4_down_2of4"]

# the other configurations reported in the `configs` object of the default run
CONFIG_SET = [("c1", "linear_128x4096"), ("c3_8of16", "down_8of16"), ("c3_2of4", "down_2of4"),
              ("c4_T1", "llama70b_decode_T1"), ("c4_T8", "llama70b_decode_T8"),
              ("c4_T32", "llama70b_decode_T32"), ("c4_T64", "llama70b_decode_T64"), ("c5", "qwen3_moe")]
DECODE_COPIES = 3  # resident weight copies the decode steps rotate through (together 1.1 GB > 256 MB MALL)


def prepare_bytes(T, K, gamma=False):
    """Algorithmic HBM bytes of one prepare: read bf16 x (2/elem) + gamma, write two code
    arrays (0.5/elem each), two scale arrays (1/32 each) and the mask (1/8)."""
    return T * K * (2 + 0.5 + 0.5 + 2 / 32 + 1 / 8) + (2 * K if gamma else 0)


def gemm_flops(T, O, K, n=2, m=4):
    """(algorithmic, executed) flops of the two-path GEMM: the backbone holds n/m of K."""
    return 2.0 * T * O * K * (1 + n / m), 4.0 * T * O * K


def gemm_bytes(T, O, K):
    """Minimum HBM bytes of one two-path GEMM: both A operands, W once, fp32 Y."""
    return 2 * T * K * 17 / 32 + O * K * 17 / 32 + 4 * T * O


def silu_bytes(T, I):
    return T * (8 * I + 2 * I)


def fused_bytes(T, I, H):
    """Minimum HBM bytes of the fused gate|up stage: both A operands, the [2I x H]
    weight, and prepare(h) written (codes, scales, mask)."""
    return 2 * T * H * 17 / 32 + 2 * I * H * 17 / 32 + T * I * (0.5 + 0.5 + 2 / 32 + 1 / 8)


def nv_prepare_bytes(T, K):
    """NVFP4 prepare: read bf16 x, write two code arrays (0.5/elem each), two E4M3
    scale arrays (1/16 each) and the mask (1/8)."""
    return T * K * (2 + 0.5 + 0.5 + 2 / 16 + 1 / 8)


def nv_gemm_bytes(T, O, K):
    """Minimum HBM bytes of the NVFP4 two-path GEMM: both A operands, W once, fp32 Y."""
    return 2 * T * K * 9 / 16 + O * K * 9 / 16 + 4 * T * O


def _to_gpu_bf16(torch, u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def _gpu_normal_bf16(torch, rows, cols, seed, sigma=0.02):
    """bf16 [rows x cols] with N(0, sigma) entries drawn on the GPU from a seeded generator."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(rows, cols, device="cuda", generator=g) * sigma).to(torch.bfloat16)


class Stage:
    """One kernel launch of a step. fn(c) launches it against weight copy c."""

    def __init__(self, name, fn, kind, bytes_=0.0, flops_alg=0.0, flops_exec=0.0, peak=FP4_PEAK_TFLOPS):
        self.name, self.fn, self.kind = name, fn, kind
        self.bytes, self.flops_alg, self.flops_exec = bytes_, flops_alg, flops_exec
        self.peak = peak  # TFLOP/s of the matrix unit the stage runs on


class Workload:
    def __init__(self, stages, tokens, cfg, copies=1, oracle=None):
        self.stages, self.tokens, self.cfg, self.copies, self.oracle = stages, tokens, cfg, copies, oracle


_DECODE_WEIGHTS = {}


def decode_weights(torch, sq, H, I, copies):
    """The Llama-3.1-70B gate|up [2I x H] and down [H x I] weights, `copies`
    independent draws (seeds 7000 + 2c, 7001 + 2c), quantised on the GPU;
    shared by the four decode workloads."""
    key = (H, I, copies)
    if key not in _DECODE_WEIGHTS:
        ws = []
        for c in range(copies):
            w_gu = sq.quantize_mxfp4(_gpu_normal_bf16(torch, 2 * I, H, 7000 + 2 * c))
            w_dn = sq.quantize_mxfp4(_gpu_normal_bf16(torch, H, I, 7001 + 2 * c))
            ws.append((w_gu, w_dn))
            torch.cuda.synchronize()
        _DECODE_WEIGHTS[key] = ws
    return _DECODE_WEIGHTS[key]


def build_workload(name, torch, sq, unfused=False):
    from synth import (array_digest, workload_down_silu, workload_linear, workload_llama70b_decode,
                       workload_llama8b_mlp, workload_qwen3_moe)
    if name == "llama8b_mlp":
        wl = workload_llama8b_mlp()
        T, H, I = wl["x"].shape[0], wl["hidden"], wl["inter"]
        x, g = _to_gpu_bf16(torch, wl["x"]), _to_gpu_bf16(torch, wl["gamma"])
        w_gu = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_gu"]))
        w_dn = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_down"]))
        eps = 1e-5  # Llama-3.1 RMSNorm epsilon
        buf = {"p1": sq.prepare(x, g, 2, 4, rms_eps=eps)}
        fa1, fe1 = gemm_flops(T, 2 * I, H)
        fa2, fe2 = gemm_flops(T, H, I)
        if unfused:
            buf["gu"] = sq.linear(buf["p1"], w_gu)
            buf["h"] = sq.silu_mul(buf["gu"])
            buf["p2"] = sq.prepare(buf["h"], None, 2, 4)
            middle = [
                Stage("gemm_gate_up", lambda c=0: sq.linear(buf["p1"], w_gu, out=buf["gu"]), "mfma",
                      gemm_bytes(T, 2 * I, H), fa1, fe1),
                Stage("silu_mul", lambda c=0: sq.silu_mul(buf["gu"], out=buf["h"]), "hbm", silu_bytes(T, I)),
                Stage("prepare_h", lambda c=0: sq.prepare(buf["h"], None, 2, 4, out=buf["p2"]), "hbm",
                      prepare_bytes(T, I)),
            ]
        else:
            buf["p2"], _ = sq.linear_silu_prepare(buf["p1"], w_gu, 2, 4)
            middle = [
                Stage("gemm_gate_up_silu_prepare",
                      lambda c=0: sq.linear_silu_prepare_into(buf["p1"], w_gu, buf["p2"], 2, 4), "mfma",
                      fused_bytes(T, I, H), fa1, fe1),
            ]
        buf["y"] = sq.linear(buf["p2"], w_dn)
        stages = [Stage("prepare_x_rmsnorm", lambda c=0: sq.prepare(x, g, 2, 4, out=buf["p1"], rms_eps=eps), "hbm",
                        prepare_bytes(T, H, True) + 4 * T)] + middle + [
            Stage("gemm_down", lambda c=0: sq.linear(buf["p2"], w_dn, out=buf["y"]), "mfma", gemm_bytes(T, H, I),
                  fa2, fe2),
        ]
        cfg = {"workload": "Llama-3.1-8B MLP block, 2048-token prefill, 2:4, MXFP4, RMSNorm (1/rms and gamma) "
                           "absorbed in the first prepare",
               "tokens": T, "hidden": H, "intermediate": I, "nm": "2:4", "rms_eps": eps, "seed": 1002,
               "gate_up": "unfused (linear, silu_mul, prepare)" if unfused else "fused (linear_silu_prepare)",
               "input_sha256_16": {k: array_digest(wl[k]) for k in ("x", "gamma", "w_gu", "w_down")}}
        return Workload(stages, T, cfg, oracle="llama8b_mlp")

    if name == "linear_128x4096" or name.startswith("down_"):
        if name == "linear_128x4096":
            wl = workload_linear()
            xb, wb, n, m = wl["x"], wl["w"], 2, 4
            label = "single linear 128x4096 -> 4096, 2:4, MXFP4"
        else:
            wl = workload_down_silu()
            xb, wb = wl["x"], wl["w"]
            n, m = (8, 16) if name == "down_8of16" else (2, 4)
            label = f"down_proj 2048x14336 -> 4096, {n}:{m}, MXFP4, SiLU-gated input"
        T, K = xb.shape
        O = wb.shape[0]
        x = _to_gpu_bf16(torch, xb)
        wq = sq.quantize_mxfp4(_to_gpu_bf16(torch, wb))
        buf = {"p": sq.prepare(x, None, n, m)}
        buf["y"] = sq.linear(buf["p"], wq)
        fa, fe = gemm_flops(T, O, K, n, m)
        kind = "mfma" if T >= 1024 else "hbm"
        stages = [Stage("prepare", lambda c=0: sq.prepare(x, None, n, m, out=buf["p"]), "hbm", prepare_bytes(T, K)),
                  Stage("gemm", lambda c=0: sq.linear(buf["p"], wq, out=buf["y"]), kind, gemm_bytes(T, O, K), fa, fe)]
        cfg = {"workload": label, "tokens": T, "in_features": K, "out_features": O, "nm": f"{n}:{m}"}
        return Workload(stages, T, cfg)

    if name.startswith("nvfp4_down_"):
        # the down projection with NVFP4 operands (16-entry blocks, E4M3 block scales, fp32 tensor scales)
        from synth import bf16_to_f32
        wl = workload_down_silu()
        xb, wb = wl["x"], wl["w"]
        n, m = (8, 16) if name == "nvfp4_down_8of16" else (2, 4)
        T, K = xb.shape
        O = wb.shape[0]
        # static tensor scales amax / (6 * 448), calibrated on the host from the same data
        s_a = float(np.float32(np.abs(bf16_to_f32(xb)).max()) / np.float32(2688.0))
        s_w = float(np.float32(np.abs(bf16_to_f32(wb)).max()) / np.float32(2688.0))
        x = _to_gpu_bf16(torch, xb)
        wq = sq.quantize_nvfp4(_to_gpu_bf16(torch, wb), s_w)
        buf = {"p": sq.prepare_nvfp4(x, s_a, None, n, m)}
        buf["y"] = sq.linear_nvfp4(buf["p"], wq)
        fa, fe = gemm_flops(T, O, K, n, m)
        stages = [Stage("prepare_nvfp4", lambda c=0: sq.prepare_nvfp4(x, s_a, None, n, m, out=buf["p"]), "hbm",
                        nv_prepare_bytes(T, K)),
                  Stage("gemm_nvfp4", lambda c=0: sq.linear_nvfp4(buf["p"], wq, out=buf["y"]), "mfma",
                        nv_gemm_bytes(T, O, K), fa, fe, F16_PEAK_TFLOPS)]
        cfg = {"workload": f"down_proj 2048x14336 -> 4096, {n}:{m}, NVFP4 (GEMM on fp16 MFMA), SiLU-gated input",
               "tokens": T, "in_features": K, "out_features": O, "nm": f"{n}:{m}", "format": "nvfp4",
               "tensor_scales": {"activation": s_a, "weight": s_w}}
        return Workload(stages, T, cfg)

    if name.startswith("compact_"):
        # compressed backbone of the down projection's input: prepare, compress, expand
        wl = workload_down_silu(with_weights=False)
        xb = wl["x"]
        n, m = (8, 16) if name == "compact_8of16" else (2, 4)
        T, K = xb.shape
        x = _to_gpu_bf16(torch, xb)
        buf = {"p": sq.prepare(x, None, n, m)}
        buf["c"] = sq.compress_backbone(buf["p"], n, m)
        buf["bb"], buf["mask"] = sq.expand_backbone(buf["c"])
        meta = buf["c"].meta.shape[1]
        dense = T * K * (0.5 + 1 / 8)            # dense backbone codes + mask
        packed = T * (K / 4 + meta)              # kept codes + rank fields
        stages = [Stage("prepare", lambda c=0: sq.prepare(x, None, n, m, out=buf["p"]), "hbm", prepare_bytes(T, K)),
                  Stage("compress_backbone", lambda c=0: sq.compress_backbone(buf["p"], n, m, out=buf["c"]), "hbm",
                        dense + packed),
                  Stage("expand_backbone", lambda c=0: sq.expand_backbone(buf["c"], buf["bb"], buf["mask"]), "hbm",
                        dense + packed)]
        cfg = {"workload": f"compressed sparse backbone of the down_proj input 2048x14336, {n}:{m}", "tokens": T,
               "in_features": K, "nm": f"{n}:{m}",
               "backbone_bytes_per_element": {"dense_codes_and_mask": 0.625, "compressed": round(packed / (T * K), 4)}}
        return Workload(stages, T, cfg)

    if name.startswith("llama70b_decode_T"):
        T = int(name.split("_T")[1])
        wl = workload_llama70b_decode(T, with_weights=False)
        H, I = wl["hidden"], wl["inter"]
        x = _to_gpu_bf16(torch, wl["x"])
        ws = decode_weights(torch, sq, H, I, DECODE_COPIES)
        buf = {"p1": sq.prepare(x, None, 2, 4)}
        fa1, fe1 = gemm_flops(T, 2 * I, H)
        fa2, fe2 = gemm_flops(T, H, I)
        if unfused:
            buf["gu"] = sq.linear(buf["p1"], ws[0][0])
            buf["h"] = sq.silu_mul(buf["gu"])
            buf["p2"] = sq.prepare(buf["h"], None, 2, 4)
            middle = [
                Stage("gemm_gate_up", lambda c=0: sq.linear(buf["p1"], ws[c][0], out=buf["gu"]), "hbm",
                      gemm_bytes(T, 2 * I, H), fa1, fe1),
                Stage("silu_mul", lambda c=0: sq.silu_mul(buf["gu"], out=buf["h"]), "hbm", silu_bytes(T, I)),
                Stage("prepare_h", lambda c=0: sq.prepare(buf["h"], None, 2, 4, out=buf["p2"]), "hbm",
                      prepare_bytes(T, I)),
            ]
        else:
            buf["p2"], _ = sq.linear_silu_prepare(buf["p1"], ws[0][0], 2, 4)
            middle = [
                Stage("gemm_gate_up_silu_prepare",
                      lambda c=0: sq.linear_silu_prepare_into(buf["p1"], ws[c][0], buf["p2"], 2, 4), "hbm",
                      fused_bytes(T, I, H), fa1, fe1),
            ]
        buf["y"] = sq.linear(buf["p2"], ws[0][1])
        stages = [Stage("prepare_x", lambda c=0: sq.prepare(x, None, 2, 4, out=buf["p1"]), "hbm",
                        prepare_bytes(T, H))] + middle + [
            Stage("gemm_down", lambda c=0: sq.linear(buf["p2"], ws[c][1], out=buf["y"]), "hbm", gemm_bytes(T, H, I),
                  fa2, fe2),
        ]
        cfg = {"workload": f"Llama-3.1-70B MLP decode, {T} tokens, 2:4, MXFP4", "tokens": T, "hidden": H,
               "intermediate": I, "nm": "2:4",
               "gate_up": "unfused (linear, silu_mul, prepare)" if unfused else "fused (linear_silu_prepare)",
               "weight_copies": DECODE_COPIES,
               "weights": "N(0, 0.02) drawn on the GPU (torch generator seeds 7000 + 2c, 7001 + 2c), MXFP4"}
        return Workload(stages, T, cfg, copies=DECODE_COPIES)

    if name == "qwen3_moe":
        wl = workload_qwen3_moe(with_weights=False)
        E, I, H = wl["experts"], wl["inter"], wl["hidden"]
        P = len(wl["a_rows"])
        tokens = wl["x"].shape[0]
        x = _to_gpu_bf16(torch, wl["x"])
        w_gu = sq.quantize_mxfp4(_gpu_normal_bf16(torch, E * 2 * I, H, 5005).view(E, 2 * I, H))
        w_dn = sq.quantize_mxfp4(_gpu_normal_bf16(torch, E * H, I, 5006).view(E, H, I))
        seg = torch.from_numpy(wl["seg_offsets"]).cuda()
        rows = torch.from_numpy(wl["a_rows"]).cuda()
        buf = {"p1": sq.prepare(x, None, 2, 4)}
        fa1, fe1 = gemm_flops(P, 2 * I, H)
        fa2, fe2 = gemm_flops(P, H, I)
        gu_in_bytes = 2 * P * H * 17 / 32 + E * 2 * I * H * 17 / 32  # gathered A of both paths + all experts' W
        if unfused:
            buf["gu"] = sq.linear_grouped(buf["p1"], w_gu, seg, rows)
            buf["h"] = sq.silu_mul(buf["gu"])
            buf["p2"] = sq.prepare(buf["h"], None, 2, 4)
            middle = [
                Stage("grouped_gate_up", lambda c=0: sq.linear_grouped(buf["p1"], w_gu, seg, rows, out=buf["gu"]),
                      "hbm", gu_in_bytes + 4 * P * 2 * I, fa1, fe1),
                Stage("silu_mul", lambda c=0: sq.silu_mul(buf["gu"], out=buf["h"]), "hbm", silu_bytes(P, I)),
                Stage("prepare_pairs", lambda c=0: sq.prepare(buf["h"], None, 2, 4, out=buf["p2"]), "hbm",
                      prepare_bytes(P, I)),
            ]
        else:
            buf["p2"], _ = sq.linear_grouped_silu_prepare(buf["p1"], w_gu, seg, rows, 2, 4)
            middle = [
                Stage("grouped_gate_up_silu_prepare",
                      lambda c=0: sq.linear_grouped_silu_prepare(buf["p1"], w_gu, seg, rows, 2, 4, out=buf["p2"]),
                      "hbm", gu_in_bytes + prepare_bytes(P, I) - 2 * P * I, fa1, fe1),
            ]
        buf["y"] = sq.linear_grouped(buf["p2"], w_dn, seg, None)
        from synth import moe_combine_index
        k = P // tokens
        cidx, cw = moe_combine_index(wl["a_rows"], wl["weight_of_pair"], tokens, k)
        cidx, cw = torch.from_numpy(cidx).cuda(), torch.from_numpy(cw).cuda()
        buf["out"] = sq.moe_combine(buf["y"], cidx, cw, bf16=True)
        stages = [
            Stage("prepare_tokens", lambda c=0: sq.prepare(x, None, 2, 4, out=buf["p1"]), "hbm",
                  prepare_bytes(tokens, H))
        ] + middle + [
            Stage("grouped_down", lambda c=0: sq.linear_grouped(buf["p2"], w_dn, seg, None, out=buf["y"]), "hbm",
                  2 * P * I * 17 / 32 + E * H * I * 17 / 32 + 4 * P * H, fa2, fe2),
            Stage("moe_combine", lambda c=0: sq.moe_combine(buf["y"], cidx, cw, out=buf["out"], bf16=True), "hbm",
                  4 * P * H + 2 * tokens * H + 8 * P),
        ]
        cfg = {"workload": "Qwen3-30B-A3B MoE expert layer, 4096 tokens, top-8 of 128, 2:4, MXFP4, weighted "
                           "combine to bf16 tokens",
               "tokens": tokens, "pairs": P, "experts": E, "hidden": H, "intermediate": I, "nm": "2:4",
               "gate_up": "unfused (linear_grouped, silu_mul, prepare)" if unfused
               else "fused (linear_grouped_silu_prepare)",
               "weights": "N(0, 0.02) drawn on the GPU (torch generator seeds 5005, 5006), MXFP4"}
        return Workload(stages, tokens, cfg)

    raise SystemExit(f"unknown workload {name}; choose from {WORKLOADS}")


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------

def capture_step_graphs(torch, wl):
    """One HIP graph per weight copy holding the whole step, captured after
    warm-up. The library enqueues kernel launches only, so the graphs hold
    kernel nodes only; inside a graph the kernels run back to back."""
    graphs = []
    for c in range(wl.copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in wl.stages:
                s.fn(c)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_step_graphs(torch, graphs, steps):
    """The timed region: K whole-step graph replays back to back (weight copies
    rotated), one HIP event recorded on the launch stream before the first and
    one after the last (an event between replays would itself add tens of us to
    each step). Returns (ms per step from the wall clock, ms per step from the
    two events)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for k in range(steps):
        graphs[k % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return 1e3 * wall / steps, a.elapsed_time(b) / steps


def settle(torch, graphs, seconds):
    """Untimed replays of the step for `seconds`: the GPU's power management
    raises clocks above their sustained level for the first milliseconds of a
    load and throttles after that, so the timed region starts only once the
    clocks have reached the sustained state."""
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            graphs[k % len(graphs)].replay()
            k += 1
        torch.cuda.synchronize()


def time_stages_back_to_back(torch, wl, launches=10, reps=5):
    """Per-stage kernel time as it runs inside a step graph: for each stage a
    graph of `launches` back-to-back launches of that stage alone (weight copies
    rotated launch by launch), replayed `reps` times with HIP events around each
    replay; returns the median per-launch ms of each stage."""
    out = []
    for s in wl.stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(launches):
                s.fn(r % wl.copies)
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for r in range(reps):
            g.replay()
            ev[r + 1].record()
        torch.cuda.synchronize()
        out.append(float(np.median([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)])) / launches)
        del g
    return out


def time_eager(torch, wl, steps):
    """K eager steps with events between the stages: (ms per step, [median ms per stage])."""
    n = len(wl.stages)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        c = k % wl.copies
        ev[k][0].record()
        for i, s in enumerate(wl.stages):
            s.fn(c)
            ev[k][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = [float(np.median([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)])) for i in range(n)]
    return 1e3 * wall / steps, stage_ms


def warm(torch, wl, steps):
    for k in range(steps):
        for s in wl.stages:
            s.fn(k % wl.copies)
    torch.cuda.synchronize()


def stage_breakdown(stages, stage_ms):
    out = {}
    for s, ms in zip(stages, stage_ms):
        d = {"us": round(ms * 1e3, 2)}
        if s.bytes:
            d["GB/s"] = round(s.bytes / (ms * 1e-3) / 1e9, 1)
            d["hbm_frac"] = round(d["GB/s"] / HBM_PEAK_GBS, 4)
        if s.flops_alg:
            d["TFLOP/s_alg"] = round(s.flops_alg / (ms * 1e-3) / 1e12, 1)
            d["TFLOP/s_exec"] = round(s.flops_exec / (ms * 1e-3) / 1e12, 1)
            d["mfma_frac_alg"] = round(d["TFLOP/s_alg"] / s.peak, 4)
        out[s.name] = d
    return out


def roofline_of(stage, ms):
    """Roofline object of a stage from its duration (algorithmic work / time)."""
    if stage.kind == "mfma":
        ach = stage.flops_alg / (ms * 1e-3) / 1e12
        return {"kernel": stage.name, "bound": "mfma", "achieved": round(ach, 1), "peak": stage.peak,
                "unit": "TFLOP/s", "frac": round(ach / stage.peak, 4), "us_per_launch": round(ms * 1e3, 2)}
    ach = stage.bytes / (ms * 1e-3) / 1e9
    return {"kernel": stage.name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "us_per_launch": round(ms * 1e3, 2)}


# ---------------------------------------------------------------------------
# Traffic records, calibration, context measurements
# ---------------------------------------------------------------------------

KERNEL_SOURCES = {"gemm": ["gemm.hip"], "prepare": ["prepare.hip"], "silu": ["glue.hip", "silu.h"],
                  "grouped": ["gemm.hip"], "compact": ["compact.hip"], "nvfp4": ["nvfp4.hip"]}
SHARED_HEADERS = ["sharq_device.h", "prepare_block.h", "prepare_io.h", "sort_network.h", "silu.h"]


def source_digest(stage_name):
    """sha256 over the HIP sources that implement a stage and the device headers
    they include (ties recorded counters to a kernel version)."""
    import hashlib
    key = "nvfp4" if "nvfp4" in stage_name else "gemm" if "gemm" in stage_name or "grouped" in stage_name else (
        "silu" if "silu" in stage_name else "compact" if "backbone" in stage_name else "prepare")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[key] + SHARED_HEADERS:
        with open(os.path.join(ROOT, "activation_sparsity_fp4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload, stage_name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (profiles/traffic.json),
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(f"{workload}/{stage_name}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(stage_name):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(n_bytes, steps):
    """Device-to-device copy of n_bytes, repeated: the reference for counter scaling."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n_bytes, "steps": steps}), flush=True)


def copy_rate(torch, n_bytes=1 << 30, reps=10):
    """Achieved HBM GB/s of a plain device-to-device copy (read + write bytes
    over time, median of reps): the practical ceiling of a mixed read/write
    stream, reported beside the 8 TB/s datasheet peak."""
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del src, dst
    return round(2 * n_bytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)


def mfma_sustained_rate(torch, reps=5, unit="fp4"):
    """TFLOP/s of the scaled FP4 MFMA (unit "fp4") or the fp16 MFMA (unit
    "f16") this GPU sustains on register operands with random bit patterns (no
    memory traffic; libsharq_calib.so, built beside the library): the rate a
    GEMM can reach once the power-limited clock is taken into account,
    reported beside the published peak."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "activation_sparsity_fp4_amd", "libsharq_calib.so"))
    fn = lib.sharq_calib_mfma_fp4 if unit == "fp4" else lib.sharq_calib_mfma_f16
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(0)
    blocks, iters = 2 * props.multi_processor_count, 4000
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    flops = blocks * 4 * iters * 8 * 2.0 * 32 * 32 * (64 if unit == "fp4" else 16)
    ts = []
    for k in range(reps + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        if fn(blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("MFMA calibration launch failed")
        b.record()
        torch.cuda.synchronize()
        if k >= 2:
            ts.append(a.elapsed_time(b))
    return round(flops / (float(np.median(ts)) * 1e-3) / 1e12, 1)


def cold_cache_times(torch, wl, steps):
    """Per-stage times with the caches cold: before each step a read of a
    1 GiB buffer evicts L2 and the 256 MB MALL, so every stage reads its
    inputs from HBM. The sweep reads rather than writes: a write would leave
    the caches full of dirty lines whose write-back would then be charged to
    the first stages. Returns (ms per step, {stage: median us})."""
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    n = len(wl.stages)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    for k in range(steps):
        scratch.amax()
        events[k][0].record()
        for i, s in enumerate(wl.stages):
            s.fn(k % wl.copies)
            events[k][i + 1].record()
    torch.cuda.synchronize()
    step_ms = float(np.median([events[k][0].elapsed_time(events[k][n]) for k in range(steps)]))
    us = {s.name: round(1e3 * float(np.median([events[k][i].elapsed_time(events[k][i + 1])
                                               for k in range(steps)])), 2)
          for i, s in enumerate(wl.stages)}
    del scratch
    return step_ms, us


def run_config(torch, sq, name, steps, warmup):
    """One of the other workloads, timed as the headline: whole-step graph
    replays (weight copies rotated where the workload has several) for
    tokens/s, per-stage back-to-back graphs for the stage times and the
    roofline of the dominant stage."""
    wl = build_workload(name, torch, sq)
    warm(torch, wl, warmup)
    graphs = capture_step_graphs(torch, wl)
    time_step_graphs(torch, graphs, max(2, warmup))
    settle(torch, graphs, 0.2)
    ms_step, ev_step = time_step_graphs(torch, graphs, steps)
    del graphs
    stage_ms = time_stages_back_to_back(torch, wl)
    dom = int(np.argmax(stage_ms))
    out = {"workload": wl.cfg["workload"], "tokens": wl.tokens,
           "tokens_per_s": round(wl.tokens / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
           "gpu_ms_per_step": round(ev_step, 4), "stages": stage_breakdown(wl.stages, stage_ms),
           "roofline": roofline_of(wl.stages[dom], stage_ms[dom])}
    traffic = recorded_traffic(name, wl.stages[dom].name)
    if traffic is not None:
        out["roofline"]["traffic"] = traffic
        out["roofline"]["algorithmic_bytes"] = round(wl.stages[dom].bytes)
    if wl.copies > 1:
        out["weight_copies_rotated"] = wl.copies
    del wl
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# CPU oracle baseline (a child process that never touches the GPU)
# ---------------------------------------------------------------------------

def _quantize_rows(w):
    from oracle import quantize_weight_ref
    return quantize_weight_ref(w)


def _oracle_weights(w, workers):
    """quantize_weight_ref over row chunks in a process pool (the oracle is
    row-independent; this only spreads the one-off set-up over the cores)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    chunks = np.array_split(w, max(1, workers * 2))
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork")) as ex:
        parts = list(ex.map(_quantize_rows, chunks))
    return np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts])


def cpu_baseline_child(workload):
    """Times the NumPy/float64 oracle of the headline chain on the host:
    prepare stages and fp64 GEMM stages separately, on two row samples, and
    extrapolates linearly (a fixed cost per call, such as dequantising W, plus
    a per-token cost) to the full batch. Weights are quantised by the oracle
    beforehand, outside the timed calls. Prints one JSON object."""
    from oracle import linear_ref, prepare_ref, silu_mul_ref
    from synth import workload_llama8b_mlp
    if workload != "llama8b_mlp":
        print(json.dumps(None))
        return
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(cores, user_api="blas")
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_name = blas[0].get("internal_api", "?") if blas else "?"
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:
        blas_name, threads = "?", cores
    wl = workload_llama8b_mlp()
    T, I = wl["x"].shape[0], wl["inter"]
    t0 = time.perf_counter()
    wgc, wgs = _oracle_weights(wl["w_gu"], min(cores, 16))
    wdc, wds = _oracle_weights(wl["w_down"], min(cores, 16))
    setup_s = time.perf_counter() - t0

    def run(rows):
        t = {}
        a = time.perf_counter()
        p1 = prepare_ref(wl["x"][:rows], wl["gamma"], 2, 4, rms_eps=1e-5)
        b = time.perf_counter()
        gu, _ = linear_ref(p1["bb_codes"], p1["bb_scales"], p1["res_codes"], p1["res_scales"], wgc, wgs)
        c = time.perf_counter()
        h = silu_mul_ref(gu.astype(np.float32), I)
        p2 = prepare_ref(h, None, 2, 4)
        d = time.perf_counter()
        linear_ref(p2["bb_codes"], p2["bb_scales"], p2["res_codes"], p2["res_scales"], wdc, wds)
        e = time.perf_counter()
        t["prepare"] = (b - a) + (d - c)
        t["gemm"] = (c - b) + (e - d)
        return t

    r1, r2 = 64, 256
    t1, t2 = run(r1), run(r2)
    est = {}
    for k in ("prepare", "gemm"):
        per = max((t2[k] - t1[k]) / (r2 - r1), 0.0)
        fixed = max(t1[k] - per * r1, 0.0)
        est[k] = {"s_per_token": per, "fixed_s": fixed, "full_batch_s": fixed + per * T}
    full = est["prepare"]["full_batch_s"] + est["gemm"]["full_batch_s"]
    print(json.dumps({
        "value": round(T / full, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": f"the numpy/float64 oracle of the whole chain (prepare with RMSNorm, gate|up GEMM, silu_mul, "
                  f"prepare(h), down GEMM) on the first {r1} and first {r2} of {T} tokens, timed per stage kind; "
                  f"value = {T} tokens over the linear extrapolation (fixed + per-token cost) of both to the "
                  f"full batch; oracle weight quantisation done beforehand ({setup_s:.1f} s, not timed)",
        "prepare_s_sample": [round(t1["prepare"], 3), round(t2["prepare"], 3)],
        "gemm_s_sample": [round(t1["gemm"], 3), round(t2["gemm"], 3)],
        "prepare_tokens_per_s": round(T / est["prepare"]["full_batch_s"], 2),
        "gemm_tokens_per_s": round(T / est["gemm"]["full_batch_s"], 2),
        "blas": {"library": blas_name, "threads": threads}}), flush=True)


def cpu_baseline(workload, timeout_s=600):
    """Runs cpu_baseline_child in a child process (it never initialises the GPU)."""
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--workload", workload]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout_s, cwd=ROOT)
    except subprocess.TimeoutExpired:
        return {"error": f"oracle timing exceeded {timeout_s} s"}
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1] if r.stderr.strip() else f"exit {r.returncode}"}
    return json.loads(r.stdout.strip().splitlines()[-1])


# ---------------------------------------------------------------------------

def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_mlp", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' `configs` object")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps per workload in `configs`")
    ap.add_argument("--unfused", action="store_true",
                    help="run gate|up, silu_mul and prepare(h) as three kernels")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed step replays before the timed region (clocks reach their sustained "
                         "state)")
    ap.add_argument("--profile-stage", default=None,
                    help="run only this stage, eagerly, in warmup and timing (per-kernel profiling; not a step)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache stage timing")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a device copy of this many bytes (reference for counter scaling)")
    ap.add_argument("--calib", choices=["fp4", "f16"], default=None,
                    help="only run the MFMA rate calibration kernel (reference for clock and MFMA-busy counters)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.cpu_baseline_child:
        cpu_baseline_child(args.workload)
        return

    import torch
    import activation_sparsity_fp4_amd as sq
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs the GPU")
    torch.cuda.init()
    if args.calib:
        print(json.dumps({"calib": args.calib, "TFLOP/s": mfma_sustained_rate(torch, unit=args.calib)}), flush=True)
        return
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return
    log(f"building inputs for {args.workload}")
    wl = build_workload(args.workload, torch, sq, args.unfused)
    torch.cuda.synchronize()
    profiling = args.profile_stage is not None
    if profiling:
        wl.stages = [s for s in wl.stages if s.name == args.profile_stage]
        if not wl.stages:
            raise SystemExit(f"no stage {args.profile_stage!r} in workload {args.workload}")

    warm(torch, wl, args.warmup)
    eager_ms, eager_stage_ms = time_eager(torch, wl, args.steps)
    log(f"warmup and eager pass done ({eager_ms:.4f} ms per step); timing {args.steps} steps")

    if args.eager or profiling:
        ms_per_step, stage_ms = time_eager(torch, wl, args.steps)
        gpu_ms_per_step = None
        timing = "eager launches, HIP events between the stages"
    else:
        graphs = capture_step_graphs(torch, wl)
        time_step_graphs(torch, graphs, max(2, args.warmup))
        settle(torch, graphs, args.settle)
        ms_per_step, gpu_ms_per_step = time_step_graphs(torch, graphs, args.steps)
        del graphs
        stage_ms = time_stages_back_to_back(torch, wl)
        timing = (f"after {args.warmup} warm-up steps and {args.settle} s of untimed replays (sustained clocks), "
                  "timed region: whole-step HIP graph replays (kernel nodes only), HIP events around the region; "
                  "stage times: a graph of 10 back-to-back launches of each stage, HIP events around its replays")
    log(f"timed region done ({ms_per_step:.4f} ms per step)")

    dom_i = int(np.argmax(stage_ms))
    dom = wl.stages[dom_i]
    roof = roofline_of(dom, stage_ms[dom_i])
    roof["traffic"] = recorded_traffic(args.workload, dom.name)
    if roof["traffic"] is not None:
        roof["traffic_unit"] = "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        roof["algorithmic_bytes"] = round(dom.bytes)
    if dom.kind == "mfma" and not profiling and not args.no_cold:
        # context: the MFMA rate this GPU sustains with random operands (power-limited clock), and the
        # kernel's executed (dense-masked) rate as a fraction of it
        sustained = mfma_sustained_rate(torch, unit="fp4" if dom.peak == FP4_PEAK_TFLOPS else "f16")
        roof["sustained_mfma_TFLOPs"] = sustained
        roof["frac_exec_of_sustained"] = round(dom.flops_exec / (stage_ms[dom_i] * 1e-3) / 1e12 / sustained, 4)
        roof["frac_alg_of_sustained"] = round(dom.flops_alg / (stage_ms[dom_i] * 1e-3) / 1e12 / sustained, 4)

    line = {
        "metric": "SharQ linear tokens/s (prepare GB/s and FP4 GEMM TFLOP/s as fractions of MI355X peak)",
        "value": round(wl.tokens / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.cfg.get("format", "mxfp4"), "data": "synthetic", "config": wl.cfg,
        "timing": timing, "roofline": roof, "stages": stage_breakdown(wl.stages, stage_ms),
        "stage_sum_us": round(1e3 * sum(stage_ms), 2),
        "gpu_ms_per_step": None if gpu_ms_per_step is None else round(gpu_ms_per_step, 4),
        "eager": {"ms_per_step": round(eager_ms, 4), "stages_us": {s.name: round(1e3 * t, 2) for s, t in
                                                                    zip(wl.stages, eager_stage_ms)}},
    }
    if not profiling and not args.no_cold:
        line["hbm_copy_GBps"] = copy_rate(torch)
        cold_ms, cold_us = cold_cache_times(torch, wl, args.steps)
        line["cold_cache"] = {"ms_per_step": round(cold_ms, 4),
                              "tokens_per_s": round(wl.tokens / (cold_ms * 1e-3), 1), "stages_us": cold_us,
                              "note": "L2 and MALL evicted by a 1 GiB read before each eager step; medians; "
                                      "not the timed region"}
    if profiling:
        line["profile_stage"] = args.profile_stage
        line["note"] = "only this stage was run; value and ms_per_step are not a full step"
    del wl
    torch.cuda.empty_cache()

    if args.workload == "llama8b_mlp" and not profiling and not args.no_configs:
        configs = {}
        for key, name in CONFIG_SET:
            log(f"config {key}: {name}")
            configs[key] = run_config(torch, sq, name, args.config_steps, 3)
        line["configs"] = configs
        _DECODE_WEIGHTS.clear()
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline and not profiling and args.workload == "llama8b_mlp":
        log("timing the CPU oracle in a child process")
        line["cpu_baseline"] = cpu_baseline(args.workload)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
