"""Helpers for the GPU parity tests: host <-> device copies and the Y tolerance."""

import numpy as np

TOL_REL = 1e-4
TOL_ABS = 1e-6


def torch():
    import torch as _t
    return _t


def dev():
    return torch().device("cuda:0")


def bf16_to_gpu(u16):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(u16, dtype=np.uint16).view(np.int16)).view(t.bfloat16).to(dev())


def u8_to_gpu(a):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def i32_to_gpu(a):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def f32_to_gpu(a):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def to_np(t):
    tt = torch()
    t = t.detach().cpu()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).numpy().view(np.uint16)
    return t.numpy()


def stage_major(s_rows):
    """Row-major scales [R, K/32] (the oracle's form) -> the library's stage-major
    [ceil(K/128), R, 4] layout, zero past the last block. Pure data movement."""
    s_rows = np.asarray(s_rows, dtype=np.uint8)
    R, kb = s_rows.shape
    G = (kb + 3) // 4
    pad = np.zeros((R, 4 * G), dtype=np.uint8)
    pad[:, :kb] = s_rows
    return np.ascontiguousarray(pad.reshape(R, G, 4).transpose(1, 0, 2))


def row_major(s_stage, kblocks):
    """Stage-major [G, R, 4] -> row-major [R, K/32]; checks the padding bytes are zero."""
    s_stage = np.asarray(s_stage, dtype=np.uint8)
    G, R, _ = s_stage.shape
    flat = s_stage.transpose(1, 0, 2).reshape(R, 4 * G)
    assert not flat[:, kblocks:].any(), "scale padding bytes must be zero"
    return flat[:, :kblocks]


def codes_stage_major(c_rows):
    """Row-major codes [R, K/2] (the oracle's form) -> the library's stage-major
    [ceil(K/128), R, 64] layout, zero past the last block. Pure data movement."""
    c_rows = np.asarray(c_rows, dtype=np.uint8)
    R, kh = c_rows.shape
    G = (kh + 63) // 64
    pad = np.zeros((R, 64 * G), dtype=np.uint8)
    pad[:, :kh] = c_rows
    return np.ascontiguousarray(pad.reshape(R, G, 64).transpose(1, 0, 2))


def codes_row_major(c_stage, kbytes):
    """Stage-major codes [G, R, 64] -> row-major [R, K/2]; checks the padding bytes are zero."""
    c_stage = np.asarray(c_stage, dtype=np.uint8)
    G, R, _ = c_stage.shape
    flat = c_stage.transpose(1, 0, 2).reshape(R, 64 * G)
    assert not flat[:, kbytes:].any(), "code padding bytes must be zero"
    return flat[:, :kbytes]


def w_to_gpu(wc, ws):
    """Upload an oracle-quantised weight (row-major codes [O, K/2] and scales
    [O, K/32], or stacks of them over experts) in the library's layout."""
    import activation_sparsity_fp4_amd as sq
    ws = np.asarray(ws)
    wc = np.asarray(wc)
    K = 2 * wc.shape[-1]
    if ws.ndim == 3:
        return sq.MXFP4(u8_to_gpu(np.stack([codes_stage_major(x) for x in wc])),
                        u8_to_gpu(np.stack([stage_major(x) for x in ws])), K)
    return sq.MXFP4(u8_to_gpu(codes_stage_major(wc)), u8_to_gpu(stage_major(ws)), K)


def w_scales_rows(wq_scales, kblocks):
    """GPU weight scales [G, O, 4] -> row-major [O, K/32]."""
    return row_major(to_np(wq_scales), kblocks)


def w_codes_rows(wq_codes, kbytes):
    """GPU weight codes [G, O, 64] -> row-major [O, K/2]."""
    return codes_row_major(to_np(wq_codes), kbytes)


def oracle_prepared(out):
    """Upload an oracle prepare result as the GPU's Prepared tuple."""
    import activation_sparsity_fp4_amd as sq
    K = 2 * out["bb_codes"].shape[1]
    return sq.Prepared(u8_to_gpu(codes_stage_major(out["bb_codes"])), u8_to_gpu(stage_major(out["bb_scales"])),
                       u8_to_gpu(codes_stage_major(out["res_codes"])), u8_to_gpu(stage_major(out["res_scales"])),
                       None, K)


def assert_prepare_equal(got, want, rows=None):
    """Bit-exact comparison of a GPU Prepared against an oracle dict (optionally on a row subset)."""
    for name in ("bb_codes", "bb_scales", "res_codes", "res_scales", "mask"):
        g = getattr(got, name)
        if g is None:
            continue
        g = to_np(g)
        if name.endswith("scales"):
            g = row_major(g, want[name].shape[1])
        elif name.endswith("codes"):
            g = codes_row_major(g, want[name].shape[1])
        if rows is not None:
            g = g[rows]
        w = want[name]
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            r, c = bad[0]
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at row {r} col {c}: "
                                 f"gpu {g[r, c]:#x} oracle {w[r, c]:#x}")


def assert_y_close(y_gpu, y_ref, bound):
    """|Y_gpu - Y_ref| <= 1e-4 * sum_k |a_k w_k| + 1e-6 elementwise."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = TOL_REL * bound + TOL_ABS
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} of {bad.size} outside tolerance; first {tuple(i)}: gpu {y_gpu[tuple(i)]} "
                             f"ref {y_ref[tuple(i)]} tol {tol[tuple(i)]}")
    return float((err / np.maximum(tol, 1e-30)).max())


def assert_bf16_close(h, want):
    """bf16 outputs of fp32 math against the correctly rounded value: within one
    bf16 ulp (same sign), or both below 2^-126 in magnitude, where fp32
    intermediate results (exp overflow in silu) legitimately flush to zero."""
    from synth import bf16_to_f32
    h = np.asarray(h, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    diff = np.abs(h.astype(np.int32) - want.astype(np.int32))
    same_sign = (h >> 15) == (want >> 15)
    tiny = (np.abs(bf16_to_f32(h)) < 2.0 ** -126) & (np.abs(bf16_to_f32(want)) < 2.0 ** -126)
    ok = ((diff <= 1) & same_sign) | tiny
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{(~ok).sum()} bf16 values off by more than one ulp; first {i}: "
                             f"gpu {h[i]:#06x} want {want[i]:#06x}")


def assert_h_close(h_bits, g_ref, g_bound, u_ref, u_bound):
    """A fused gate|up kernel's h = bf16(silu(g) * u), computed on the GPU's own
    fp32 g and u, against the oracle's float64 g and u (linear_ref and its
    bound B for the gate and the up column).

    The GPU's g and u lie within tau = 1e-4 B + 1e-6 of the oracle's (the Y
    tolerance). |d silu / dg| <= 1.1 everywhere (its extremes are about 1.0998
    and -0.0998), so silu(g) * u moves by at most
        delta = 1.1 (|u| + tau_u) tau_g + (|silu(g)| + 1.1 tau_g) tau_u;
    rounding to bf16 (and the fp32 arithmetic before it) adds at most one bf16
    ulp of the result's magnitude, and fp32 intermediates may flush below
    2^-126. Passes when |h - silu(g_ref) u_ref| <= delta + ulp + 2^-126."""
    from synth import bf16_to_f32
    h = bf16_to_f32(np.asarray(h_bits, dtype=np.uint16)).astype(np.float64)
    g = np.asarray(g_ref, dtype=np.float64)
    u = np.asarray(u_ref, dtype=np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    f = silu * u
    tg = TOL_REL * np.asarray(g_bound, dtype=np.float64) + TOL_ABS
    tu = TOL_REL * np.asarray(u_bound, dtype=np.float64) + TOL_ABS
    delta = 1.1 * (np.abs(u) + tu) * tg + (np.abs(silu) + 1.1 * tg) * tu
    mag = np.maximum(np.abs(f) + delta, 2.0 ** -126)
    ulp = np.ldexp(1.0, np.frexp(mag)[1] - 1 - 7)
    tol = delta + ulp + 2.0 ** -126
    err = np.abs(h - f)
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{bad.sum()} of {bad.size} h values outside tolerance; first {i}: gpu {h[i]} "
                             f"oracle silu(g)*u {f[i]} (g {g[i]}, u {u[i]}) tol {tol[i]}")
    return float((err / tol).max())
