#!/usr/bin/env python3
"""Benchmark of the SharQ linear hot path on one MI355X.

Default workload: a Llama-3.1-8B-shaped MLP block at 2048-token prefill, 2:4,
MXFP4, the RMSNorm (per-row 1/rms and gamma) absorbed in the first prepare:
    prepare(rmsnorm(x)) -> fused [two-path GEMM gate|up [28672 x 4096] ->
    silu(gate) * up -> prepare(h)] -> two-path GEMM down [4096 x 14336]
One step = one pass of that chain over 2048 tokens. Inputs are seeded synthetic
data resident in HBM before the timed region; weights are quantised once on
the GPU (not timed).

Prints ONE JSON line with tokens/s, the per-stage breakdown (HIP events on the
launch stream), the roofline of the dominant kernel and the CPU oracle timed on
a bounded sample of the same workload. Other workloads: --workload NAME.
"""

from __future__ import annotations

import argparse
import json
import os
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


def _to_gpu_bf16(torch, u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def nv_prepare_bytes(T, K):
    """NVFP4 prepare: read bf16 x, write two code arrays (0.5/elem each), two E4M3
    scale arrays (1/16 each) and the mask (1/8)."""
    return T * K * (2 + 0.5 + 0.5 + 2 / 16 + 1 / 8)


def nv_gemm_bytes(T, O, K):
    """Minimum HBM bytes of the NVFP4 two-path GEMM: both A operands, W once, fp32 Y."""
    return 2 * T * K * 9 / 16 + O * K * 9 / 16 + 4 * T * O


class Stage:
    def __init__(self, name, fn, kind, bytes_=0.0, flops_alg=0.0, flops_exec=0.0, peak=FP4_PEAK_TFLOPS):
        self.name, self.fn, self.kind = name, fn, kind
        self.bytes, self.flops_alg, self.flops_exec = bytes_, flops_alg, flops_exec
        self.peak = peak  # TFLOP/s of the matrix unit the stage runs on


def build_workload(name, torch, sq, unfused=False):
    """Returns (stages, tokens_per_step, config dict, oracle sample fn)."""
    from synth import (workload_down_silu, workload_linear, workload_llama70b_decode, workload_llama8b_mlp,
                       workload_qwen3_moe)
    if name == "llama8b_mlp":
        wl = workload_llama8b_mlp()
        T, H, I = wl["x"].shape[0], wl["hidden"], wl["inter"]
        x, g = _to_gpu_bf16(torch, wl["x"]), _to_gpu_bf16(torch, wl["gamma"])
        w_gu = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_gu"]))
        w_dn = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_down"]))
        eps = 1e-5  # Llama-3.1 RMSNorm epsilon
        buf = {}
        buf["p1"] = sq.prepare(x, g, 2, 4, rms_eps=eps)
        fa1, fe1 = gemm_flops(T, 2 * I, H)
        fa2, fe2 = gemm_flops(T, H, I)
        if unfused:
            buf["gu"] = sq.linear(buf["p1"], w_gu)
            buf["h"] = sq.silu_mul(buf["gu"])
            buf["p2"] = sq.prepare(buf["h"], None, 2, 4)
            middle = [
                Stage("gemm_gate_up", lambda: sq.linear(buf["p1"], w_gu, out=buf["gu"]), "mfma",
                      gemm_bytes(T, 2 * I, H), fa1, fe1),
                Stage("silu_mul", lambda: sq.silu_mul(buf["gu"], out=buf["h"]), "hbm", silu_bytes(T, I)),
                Stage("prepare_h", lambda: sq.prepare(buf["h"], None, 2, 4, out=buf["p2"]), "hbm",
                      prepare_bytes(T, I)),
            ]
        else:
            buf["p2"], _ = sq.linear_silu_prepare(buf["p1"], w_gu, 2, 4)
            middle = [
                Stage("gemm_gate_up_silu_prepare",
                      lambda: sq.linear_silu_prepare_into(buf["p1"], w_gu, buf["p2"], 2, 4), "mfma",
                      fused_bytes(T, I, H), fa1, fe1),
            ]
        buf["y"] = sq.linear(buf["p2"], w_dn)
        stages = [Stage("prepare_x_rmsnorm", lambda: sq.prepare(x, g, 2, 4, out=buf["p1"], rms_eps=eps), "hbm",
                        prepare_bytes(T, H, True) + 4 * T)] + middle + [
            Stage("gemm_down", lambda: sq.linear(buf["p2"], w_dn, out=buf["y"]), "mfma", gemm_bytes(T, H, I), fa2, fe2),
        ]
        from synth import array_digest
        cfg = {"workload": "Llama-3.1-8B MLP block, 2048-token prefill, 2:4, MXFP4, RMSNorm (1/rms and gamma) "
                           "absorbed in the first prepare",
               "tokens": T, "hidden": H, "intermediate": I, "nm": "2:4", "rms_eps": eps, "seed": 1002,
               "gate_up": "unfused (linear, silu_mul, prepare)" if unfused else "fused (linear_silu_prepare)",
               "input_sha256_16": {k: array_digest(wl[k]) for k in ("x", "gamma", "w_gu", "w_down")}}

        def oracle_sample(rows):
            from oracle import linear_ref, prepare_ref, quantize_weight_ref, silu_mul_ref
            xs = wl["x"][:rows]
            t0 = time.perf_counter()
            p1 = prepare_ref(xs, wl["gamma"], 2, 4, rms_eps=1e-5)
            wc, ws = quantize_weight_ref(wl["w_gu"])
            gu, _ = linear_ref(p1["bb_codes"], p1["bb_scales"], p1["res_codes"], p1["res_scales"], wc, ws)
            h = silu_mul_ref(gu.astype(np.float32), I)
            p2 = prepare_ref(h, None, 2, 4)
            wc, ws = quantize_weight_ref(wl["w_down"])
            linear_ref(p2["bb_codes"], p2["bb_scales"], p2["res_codes"], p2["res_scales"], wc, ws)
            return time.perf_counter() - t0
        return stages, T, cfg, oracle_sample

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
        stages = [Stage("prepare", lambda: sq.prepare(x, None, n, m, out=buf["p"]), "hbm", prepare_bytes(T, K)),
                  Stage("gemm", lambda: sq.linear(buf["p"], wq, out=buf["y"]), "mfma", gemm_bytes(T, O, K), fa, fe)]
        cfg = {"workload": label, "tokens": T, "in_features": K, "out_features": O, "nm": f"{n}:{m}"}

        def oracle_sample(rows):
            from oracle import linear_ref, prepare_ref, quantize_weight_ref
            t0 = time.perf_counter()
            p = prepare_ref(xb[:rows], None, n, m)
            wc, ws = quantize_weight_ref(wb)
            linear_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], wc, ws)
            return time.perf_counter() - t0
        return stages, T, cfg, oracle_sample

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
        stages = [Stage("prepare_nvfp4", lambda: sq.prepare_nvfp4(x, s_a, None, n, m, out=buf["p"]), "hbm",
                        nv_prepare_bytes(T, K)),
                  Stage("gemm_nvfp4", lambda: sq.linear_nvfp4(buf["p"], wq, out=buf["y"]), "mfma",
                        nv_gemm_bytes(T, O, K), fa, fe, F16_PEAK_TFLOPS)]
        cfg = {"workload": f"down_proj 2048x14336 -> 4096, {n}:{m}, NVFP4 (GEMM on fp16 MFMA), SiLU-gated input",
               "tokens": T, "in_features": K, "out_features": O, "nm": f"{n}:{m}", "format": "nvfp4",
               "tensor_scales": {"activation": s_a, "weight": s_w}}

        def oracle_sample(rows):
            from oracle import linear_nvfp4_ref, prepare_nvfp4_ref, quantize_weight_nvfp4_ref
            t0 = time.perf_counter()
            p = prepare_nvfp4_ref(xb[:rows], None, n, m, s_a)
            wc, ws = quantize_weight_nvfp4_ref(wb, s_w)
            linear_nvfp4_ref(p["bb_codes"], p["bb_scales"], p["res_codes"], p["res_scales"], s_a, wc, ws, s_w)
            return time.perf_counter() - t0
        return stages, T, cfg, oracle_sample

    if name.startswith("compact_"):
        # compressed backbone of the down projection's input: prepare, compress, expand
        wl = workload_down_silu()
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
        stages = [Stage("prepare", lambda: sq.prepare(x, None, n, m, out=buf["p"]), "hbm", prepare_bytes(T, K)),
                  Stage("compress_backbone", lambda: sq.compress_backbone(buf["p"], n, m, out=buf["c"]), "hbm",
                        dense + packed),
                  Stage("expand_backbone", lambda: sq.expand_backbone(buf["c"], buf["bb"], buf["mask"]), "hbm",
                        dense + packed)]
        cfg = {"workload": f"compressed sparse backbone of the down_proj input 2048x14336, {n}:{m}", "tokens": T,
               "in_features": K, "nm": f"{n}:{m}",
               "backbone_bytes_per_element": {"dense_codes_and_mask": 0.625, "compressed": round(packed / (T * K), 4)}}
        return stages, T, cfg, None

    if name.startswith("llama70b_decode_T"):
        T = int(name.split("_T")[1])
        wl = workload_llama70b_decode(T)
        H, I = wl["hidden"], wl["inter"]
        x = _to_gpu_bf16(torch, wl["x"])
        w_gu = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_gu"]))
        w_dn = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_down"]))
        buf = {"p1": sq.prepare(x, None, 2, 4)}
        fa1, fe1 = gemm_flops(T, 2 * I, H)
        fa2, fe2 = gemm_flops(T, H, I)
        if unfused:
            buf["gu"] = sq.linear(buf["p1"], w_gu)
            buf["h"] = sq.silu_mul(buf["gu"])
            buf["p2"] = sq.prepare(buf["h"], None, 2, 4)
            middle = [
                Stage("gemm_gate_up", lambda: sq.linear(buf["p1"], w_gu, out=buf["gu"]), "hbm",
                      gemm_bytes(T, 2 * I, H), fa1, fe1),
                Stage("silu_mul", lambda: sq.silu_mul(buf["gu"], out=buf["h"]), "hbm", silu_bytes(T, I)),
                Stage("prepare_h", lambda: sq.prepare(buf["h"], None, 2, 4, out=buf["p2"]), "hbm",
                      prepare_bytes(T, I)),
            ]
        else:
            buf["p2"], _ = sq.linear_silu_prepare(buf["p1"], w_gu, 2, 4)
            middle = [
                Stage("gemm_gate_up_silu_prepare",
                      lambda: sq.linear_silu_prepare_into(buf["p1"], w_gu, buf["p2"], 2, 4), "hbm",
                      fused_bytes(T, I, H), fa1, fe1),
            ]
        buf["y"] = sq.linear(buf["p2"], w_dn)
        stages = [Stage("prepare_x", lambda: sq.prepare(x, None, 2, 4, out=buf["p1"]), "hbm", prepare_bytes(T, H))
                  ] + middle + [
            Stage("gemm_down", lambda: sq.linear(buf["p2"], w_dn, out=buf["y"]), "hbm", gemm_bytes(T, H, I), fa2, fe2),
        ]
        cfg = {"workload": f"Llama-3.1-70B MLP decode, {T} tokens, 2:4, MXFP4", "tokens": T, "hidden": H,
               "intermediate": I, "nm": "2:4",
               "gate_up": "unfused (linear, silu_mul, prepare)" if unfused else "fused (linear_silu_prepare)"}
        return stages, T, cfg, None

    if name == "qwen3_moe":
        wl = workload_qwen3_moe()
        E, I, H = wl["experts"], wl["inter"], wl["hidden"]
        P = len(wl["a_rows"])
        tokens = wl["x"].shape[0]
        x = _to_gpu_bf16(torch, wl["x"])
        w_gu = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_gu"].reshape(E * 2 * I, H)).view(E, 2 * I, H))
        w_dn = sq.quantize_mxfp4(_to_gpu_bf16(torch, wl["w_down"].reshape(E * H, I)).view(E, H, I))
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
                Stage("grouped_gate_up", lambda: sq.linear_grouped(buf["p1"], w_gu, seg, rows, out=buf["gu"]), "hbm",
                      gu_in_bytes + 4 * P * 2 * I, fa1, fe1),
                Stage("silu_mul", lambda: sq.silu_mul(buf["gu"], out=buf["h"]), "hbm", silu_bytes(P, I)),
                Stage("prepare_pairs", lambda: sq.prepare(buf["h"], None, 2, 4, out=buf["p2"]), "hbm",
                      prepare_bytes(P, I)),
            ]
        else:
            buf["p2"], _ = sq.linear_grouped_silu_prepare(buf["p1"], w_gu, seg, rows, 2, 4)
            middle = [
                Stage("grouped_gate_up_silu_prepare",
                      lambda: sq.linear_grouped_silu_prepare(buf["p1"], w_gu, seg, rows, 2, 4, out=buf["p2"]), "hbm",
                      gu_in_bytes + prepare_bytes(P, I) - 2 * P * I, fa1, fe1),
            ]
        buf["y"] = sq.linear_grouped(buf["p2"], w_dn, seg, None)
        from synth import moe_combine_index
        k = P // tokens
        cidx, cw = moe_combine_index(wl["a_rows"], wl["weight_of_pair"], tokens, k)
        cidx, cw = torch.from_numpy(cidx).cuda(), torch.from_numpy(cw).cuda()
        buf["out"] = sq.moe_combine(buf["y"], cidx, cw, bf16=True)
        stages = [
            Stage("prepare_tokens", lambda: sq.prepare(x, None, 2, 4, out=buf["p1"]), "hbm", prepare_bytes(tokens, H))
        ] + middle + [
            Stage("grouped_down", lambda: sq.linear_grouped(buf["p2"], w_dn, seg, None, out=buf["y"]), "hbm",
                  2 * P * I * 17 / 32 + E * H * I * 17 / 32 + 4 * P * H, fa2, fe2),
            Stage("moe_combine", lambda: sq.moe_combine(buf["y"], cidx, cw, out=buf["out"], bf16=True), "hbm",
                  4 * P * H + 2 * tokens * H + 8 * P),
        ]
        cfg = {"workload": "Qwen3-30B-A3B MoE expert layer, 4096 tokens, top-8 of 128, 2:4, MXFP4, weighted "
                           "combine to bf16 tokens",
               "tokens": tokens, "pairs": P, "experts": E, "hidden": H, "intermediate": I, "nm": "2:4",
               "gate_up": "unfused (linear_grouped, silu_mul, prepare)" if unfused
               else "fused (linear_grouped_silu_prepare)"}
        return stages, tokens, cfg, None

    raise SystemExit(f"unknown workload {name}; choose from {WORKLOADS}")


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


def cpu_baseline(oracle_sample, tokens_full, budget_s=20.0):
    """Time the CPU oracle on a bounded row sample; grow the sample until it takes
    a few seconds, stop before the budget."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
        blas_name = blas[0].get("internal_api", "?") if blas else "?"
    except Exception:
        threads, blas_name = os.cpu_count() or 1, "?"
    rows, spent = 4, 0.0
    while True:
        dt = oracle_sample(rows)
        spent += dt
        if dt > budget_s / 4 or rows * 2 > tokens_full or spent + 2.5 * dt > budget_s:
            break
        rows *= 2
    return {"value": rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {tokens_full} tokens through the numpy/fp64 oracle of the same chain "
                      f"(weights quantised inside the timed call), {dt:.2f} s; BLAS {blas_name} with {threads} threads"}


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


def cold_cache_times(stages, steps, torch):
    """Per-stage times with the caches cold: before each step a read of a
    1 GiB buffer evicts L2 and the 256 MB MALL, so every stage reads its
    inputs from HBM (the timed loop runs steps back to back, where weights and
    activations that fit stay cached between steps). The sweep reads rather
    than writes: a write would leave the caches full of dirty lines whose
    write-back would then be charged to the first stages. Returns (ms per
    step, {stage: median us})."""
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    n = len(stages)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    for k in range(steps):
        scratch.amax()
        events[k][0].record()
        for i, s in enumerate(stages):
            s.fn()
            events[k][i + 1].record()
    torch.cuda.synchronize()
    step_ms = float(np.median([events[k][0].elapsed_time(events[k][n]) for k in range(steps)]))
    us = {s.name: round(1e3 * float(np.median([events[k][i].elapsed_time(events[k][i + 1]) for k in range(steps)])), 2)
          for i, s in enumerate(stages)}
    del scratch
    return step_ms, us


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_mlp", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="llama8b_mlp: run gate|up, silu_mul and prepare(h) as three kernels")
    ap.add_argument("--profile-stage", default=None,
                    help="run only this stage in warmup and timing (per-kernel profiling; not a step)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache stage timing")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a device copy of this many bytes (reference for counter scaling)")
    ap.add_argument("--calib", choices=["fp4", "f16"], default=None,
                    help="only run the MFMA rate calibration kernel (reference for clock and MFMA-busy counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import activation_sparsity_fp4_amd as sq
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs the GPU")
    torch.cuda.init()
    if args.calib:
        import torch
        print(json.dumps({"calib": args.calib, "TFLOP/s": mfma_sustained_rate(torch, unit=args.calib)}), flush=True)
        return
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return
    print(f"# building inputs for {args.workload}", file=sys.stderr, flush=True)
    stages, tokens, cfg, oracle_sample = build_workload(args.workload, torch, sq, args.unfused)
    torch.cuda.synchronize()
    if args.profile_stage:
        stages = [s for s in stages if s.name == args.profile_stage]
        if not stages:
            raise SystemExit(f"no stage {args.profile_stage!r} in workload {args.workload}")

    for _ in range(args.warmup):
        for s in stages:
            s.fn()
    torch.cuda.synchronize()

    # Stage breakdown (untimed): HIP events between all stages, medians over
    # `steps` steps; it names the dominant stage.
    n = len(stages)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev = events[k]
        ev[0].record()
        for i, s in enumerate(stages):
            s.fn()
            ev[i + 1].record()
    torch.cuda.synchronize()
    stage_ms = [float(np.median([events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps)]))
                for i in range(n)]
    dom_i = int(np.argmax(stage_ms))
    print(f"# warmup and breakdown done, timing {args.steps} steps", file=sys.stderr, flush=True)

    # Timed region: K steps back to back; HIP events (on the launch stream)
    # bracket only the dominant stage, whose live median duration feeds the
    # roofline (events between every stage would add their own gaps to the
    # step).
    dom_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for i, s in enumerate(stages):
            if i == dom_i:
                dom_ev[k][0].record()
                s.fn()
                dom_ev[k][1].record()
            else:
                s.fn()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = float(np.median([dom_ev[k][0].elapsed_time(dom_ev[k][1]) for k in range(args.steps)]))

    ms_per_step = 1e3 * wall / args.steps
    breakdown = {}
    for s, ms in zip(stages, stage_ms):
        d = {"us": round(ms * 1e3, 2)}
        if s.bytes:
            d["GB/s"] = round(s.bytes / (ms * 1e-3) / 1e9, 1)
            d["hbm_frac"] = round(d["GB/s"] / HBM_PEAK_GBS, 4)
        if s.flops_alg:
            d["TFLOP/s_alg"] = round(s.flops_alg / (ms * 1e-3) / 1e12, 1)
            d["TFLOP/s_exec"] = round(s.flops_exec / (ms * 1e-3) / 1e12, 1)
            d["mfma_frac_alg"] = round(d["TFLOP/s_alg"] / s.peak, 4)
        breakdown[s.name] = d

    # dominant kernel: the stage with the largest median duration in the breakdown;
    # achieved = its algorithmic work over its live median duration in the timed region
    dom = stages[dom_i]
    traffic = recorded_traffic(args.workload, dom.name)
    if dom.kind == "mfma":
        ach = dom.flops_alg / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": dom.name, "bound": "mfma", "achieved": round(ach, 1), "peak": dom.peak,
                "unit": "TFLOP/s", "frac": round(ach / dom.peak, 4), "traffic": traffic,
                "us_per_launch": round(dom_ms * 1e3, 2)}
    else:
        ach = dom.bytes / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dom.name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "us_per_launch": round(dom_ms * 1e3, 2)}
    if dom.kind == "mfma" and not args.profile_stage and not args.no_cold:
        # context: the MFMA rate this GPU sustains with random operands (power-limited clock), and the
        # kernel's executed (dense-masked) rate as a fraction of it
        sustained = mfma_sustained_rate(torch, unit="fp4" if dom.peak == FP4_PEAK_TFLOPS else "f16")
        roof["sustained_mfma_TFLOPs"] = sustained
        roof["frac_exec_of_sustained"] = round(dom.flops_exec / (dom_ms * 1e-3) / 1e12 / sustained, 4)
    if traffic is not None:
        roof["traffic_unit"] = "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        roof["algorithmic_bytes"] = round(dom.bytes)

    value = tokens * args.steps / wall
    line = {
        "metric": "SharQ linear tokens/s (prepare GB/s and FP4 GEMM TFLOP/s as fractions of MI355X peak)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.get("format", "mxfp4"), "data": "synthetic", "config": cfg, "roofline": roof, "stages": breakdown,
    }
    if not args.profile_stage and not args.no_cold:
        line["hbm_copy_GBps"] = copy_rate(torch)
        cold_ms, cold_us = cold_cache_times(stages, args.steps, torch)
        line["cold_cache"] = {"ms_per_step": round(cold_ms, 4), "tokens_per_s": round(tokens / (cold_ms * 1e-3), 1),
                              "stages_us": cold_us,
                              "note": "L2 and MALL evicted by a 1 GiB read before each step; medians; not the timed region"}
    if args.profile_stage:
        line["profile_stage"] = args.profile_stage
        line["note"] = "only this stage was run; value and ms_per_step are not a full step"
    if oracle_sample is not None and not args.no_cpu_baseline and not args.profile_stage:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(oracle_sample, tokens)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
