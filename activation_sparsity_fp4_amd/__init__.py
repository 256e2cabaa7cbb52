"""SharQ linear hot path for AMD MI355X (gfx950).

Thin PyTorch-facing wrappers over the C ABI in ``include/sharq.h``: they check
tensor dtypes/devices, allocate outputs with ``torch.empty`` and pass raw device
pointers and the current HIP stream. All arithmetic runs in libsharq.so.

    prep = prepare(x, gamma=None, n=2, m=4)        # x: bf16 [T, K] on the GPU
    wq = quantize_mxfp4(w)                         # w: bf16 [O, K]
    y = linear(prep, wq)                           # fp32 [T, O]
"""

from __future__ import annotations

from typing import NamedTuple, Optional

from . import _lib
from ._lib import SCRATCHFREE_MAX_BYTES, SharqError, status_string  # noqa: F401

__all__ = [
    "Prepared",
    "MXFP4",
    "prepare",
    "quantize_mxfp4",
    "linear",
    "linear_scratchfree",
    "linear_grouped",
    "linear_silu_prepare",
    "linear_silu_prepare_into",
    "linear_grouped_silu_prepare",
    "CompactBackbone",
    "compress_backbone",
    "expand_backbone",
    "moe_combine",
    "silu_mul",
    "NVPrepared",
    "NVFP4",
    "prepare_nvfp4",
    "quantize_nvfp4",
    "linear_nvfp4",
    "pack_mxfp4",
    "pack_nvfp4",
    "unpack_stage_major",
    "SharqError",
    "status_string",
]


class Prepared(NamedTuple):
    """Outputs of the prepare operator (uint8 device tensors) and K.

    Codes and scales are stage-major with G = ceil(K/128) stages of 128 K
    entries: the 16 code bytes of block b = k // 32 of row t sit at
    codes[b // 4, t, 16 * (b % 4):][:16] and its scale byte at
    scales[b // 4, t, b % 4]; blocks past K // 32 are zero."""
    bb_codes: "object"    # [G, T, 64]
    bb_scales: "object"   # [G, T, 4]
    res_codes: "object"   # [G, T, 64]
    res_scales: "object"  # [G, T, 4]
    mask: "object"        # [T, K/8] (row-major bitmap) or None
    K: int
    rms_scale: "object" = None  # fp32 [T] per-row 1/rms when the RMSNorm was absorbed


class MXFP4(NamedTuple):
    """A block-scaled FP4 tensor, stage-major: codes [G, R, 64] and scales
    [G, R, 4]; for expert weights codes [E, G, O, 64] and scales [E, G, O, 4]."""
    codes: "object"
    scales: "object"
    K: int


def stages(K: int) -> int:
    """Number of 128-entry K stages (the leading dimension of a scale tensor)."""
    return (K + 127) // 128


def _torch():
    import torch
    return torch


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _check_stage_major(codes, scales, R, K, name):
    G = stages(K)
    if tuple(codes.shape) != (G, R, 64) or tuple(scales.shape) != (G, R, 4):
        raise ValueError(f"{name}: expected stage-major codes [{G}, {R}, 64] and scales [{G}, {R}, 4], "
                         f"got {tuple(codes.shape)} and {tuple(scales.shape)}")
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError(f"{name}: codes and scales must be contiguous")


def _check_matrix(t, dtype, rows, cols, name, contiguous=False):
    """A [rows, cols] device tensor of dtype with unit column stride (and
    contiguous rows when the entry point takes no leading dimension): the
    kernels write rows x cols entries through it, so nothing smaller passes."""
    _need(t, dtype, name, 2)
    if tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name}: expected shape ({rows}, {cols}), got {tuple(t.shape)}")
    if t.stride(1) != 1 or (contiguous and not t.is_contiguous()):
        raise ValueError(f"{name} must be {'contiguous' if contiguous else 'contiguous along its rows'}")


def _check_prepared(prep):
    torch = _torch()
    for name in ("bb_codes", "res_codes", "bb_scales", "res_scales"):
        _need(getattr(prep, name), torch.uint8, name, 3)
    T = prep.bb_codes.shape[1]
    _check_stage_major(prep.bb_codes, prep.bb_scales, T, prep.K, "backbone")
    _check_stage_major(prep.res_codes, prep.res_scales, T, prep.K, "residual")
    if prep.mask is not None:
        _check_matrix(prep.mask, torch.uint8, T, prep.K // 8, "mask", contiguous=True)


def prepare(x, gamma=None, n: int = 2, m: int = 4, with_mask: bool = True, out: Optional[Prepared] = None,
            rms_eps: Optional[float] = None) -> Prepared:
    """Fused prepare: N:M mask, MXFP4 backbone, residual against it, MXFP4 residual.
    With rms_eps the whole RMSNorm (per-row 1/rms, then gamma) is absorbed
    first; the per-row scales are returned in ``rms_scale``."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous along K")
    T, K = x.shape
    if gamma is not None:
        _need(gamma, torch.bfloat16, "gamma", 1)
        if gamma.numel() != K:  # the kernels read K entries of gamma
            raise ValueError(f"gamma must hold K = {K} entries, got {gamma.numel()}")
        gamma = gamma.contiguous()
    if out is None:
        kw = dict(dtype=torch.uint8, device=x.device)
        G = stages(K)
        out = Prepared(torch.empty((G, T, 64), **kw), torch.empty((G, T, 4), **kw),
                       torch.empty((G, T, 64), **kw), torch.empty((G, T, 4), **kw),
                       torch.empty((T, K // 8), **kw) if with_mask else None, K,
                       torch.empty((T,), dtype=torch.float32, device=x.device) if rms_eps is not None else None)
    else:
        if out.K != K:
            raise ValueError("out was allocated for another K")
        _check_prepared(out)
        if out.bb_codes.shape[1] != T:
            raise ValueError("out was allocated for another number of rows")
    if rms_eps is not None:
        if out.rms_scale is None:
            raise ValueError("out has no rms_scale buffer")
        _need(out.rms_scale, torch.float32, "rms_scale", 1)
        if out.rms_scale.numel() != T or not out.rms_scale.is_contiguous():
            raise ValueError("rms_scale must be a contiguous fp32 [T] tensor")
        st = _lib.call("sharq_prepare_rms", x.data_ptr(), T, K, x.stride(0), _ptr(gamma), float(rms_eps), n, m,
                       out.rms_scale.data_ptr(), out.bb_codes.data_ptr(), out.bb_scales.data_ptr(),
                       out.res_codes.data_ptr(), out.res_scales.data_ptr(), _ptr(out.mask), _stream(x.device))
        _lib.check("sharq_prepare_rms", st)
        return out
    st = _lib.call("sharq_prepare", x.data_ptr(), T, K, x.stride(0), _ptr(gamma), n, m,
                   out.bb_codes.data_ptr(), out.bb_scales.data_ptr(), out.res_codes.data_ptr(),
                   out.res_scales.data_ptr(), _ptr(out.mask), _stream(x.device))
    _lib.check("sharq_prepare", st)
    return out


def quantize_mxfp4(x, out: Optional[MXFP4] = None) -> MXFP4:
    """Plain MXFP4 along the last axis of a bf16 [R, K] tensor (e.g. a weight
    [O, K]), or of a stack of expert weights [E, O, K] (one call per expert,
    so each expert owns a contiguous [G, O, 4] scale block)."""
    torch = _torch()
    if x.dim() == 3:
        E, R, K = x.shape
        if out is None:
            out = MXFP4(torch.empty((E, stages(K), R, 64), dtype=torch.uint8, device=x.device),
                        torch.empty((E, stages(K), R, 4), dtype=torch.uint8, device=x.device), K)
        for e in range(E):
            quantize_mxfp4(x[e], MXFP4(out.codes[e], out.scales[e], K))
        return out
    _need(x, torch.bfloat16, "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous along K")
    R, K = x.shape
    if out is None:
        out = MXFP4(torch.empty((stages(K), R, 64), dtype=torch.uint8, device=x.device),
                    torch.empty((stages(K), R, 4), dtype=torch.uint8, device=x.device), K)
    _need(out.codes, torch.uint8, "out.codes", 3)
    _need(out.scales, torch.uint8, "out.scales", 3)
    _check_stage_major(out.codes, out.scales, R, K, "out")
    st = _lib.call("sharq_quantize_mxfp4", x.data_ptr(), R, K, x.stride(0), out.codes.data_ptr(),
                   out.scales.data_ptr(), _stream(x.device))
    _lib.check("sharq_quantize_mxfp4", st)
    return out


_workspaces = {}


def _workspace(device, nbytes):
    """A device workspace of at least nbytes for split-K calls, cached per
    (device, stream) so that calls on one stream (which never overlap) share it."""
    torch = _torch()
    key = (device.index, _stream(device))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def linear(prep: Prepared, w: MXFP4, out=None, split_k: bool = True):
    """Two-path FP4 GEMM: Y = deq(backbone) W^T + deq(residual) W^T, fp32 [T, O].
    With split_k, K is split over a cached workspace (sharq_linear_ws) where
    the library's plan expects it to be faster (too few output tiles to fill
    the GPU, K long enough); the result is deterministic."""
    torch = _torch()
    _check_prepared(prep)
    _need(w.codes, torch.uint8, "w.codes", 3)
    _need(w.scales, torch.uint8, "w.scales", 3)
    T, K = prep.bb_codes.shape[1], prep.K
    O = w.codes.shape[1]
    if w.K != K:
        raise ValueError("weight K does not match the activation K")
    _check_stage_major(w.codes, w.scales, O, K, "w")
    if out is None:
        out = torch.empty((T, O), dtype=torch.float32, device=prep.bb_codes.device)
    _check_matrix(out, torch.float32, T, O, "out")
    nbytes = _lib.call("sharq_linear_workspace_bytes", T, O, K) if split_k else 0
    if nbytes > 0:
        ws = _workspace(out.device, nbytes)
        st = _lib.call("sharq_linear_ws", prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(),
                       prep.res_codes.data_ptr(), prep.res_scales.data_ptr(), w.codes.data_ptr(), w.scales.data_ptr(),
                       T, O, K, out.data_ptr(), out.stride(0), ws.data_ptr(), ws.numel(), _stream(out.device))
        _lib.check("sharq_linear_ws", st)
        return out
    st = _lib.call("sharq_linear", prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(), prep.res_codes.data_ptr(),
                   prep.res_scales.data_ptr(), w.codes.data_ptr(), w.scales.data_ptr(), T, O, K,
                   out.data_ptr(), out.stride(0), _stream(out.device))
    _lib.check("sharq_linear", st)
    return out


def linear_scratchfree(prep: Prepared, w: MXFP4, out):
    """linear() with any K split's partials in the library's static scratch
    array instead of a workspace: nothing is allocated, so `out` (fp32
    [T, O]) is required. Raises SharqError (SHARQ_ESCRATCH) when the split
    plan needs more than SCRATCHFREE_MAX_BYTES. Calls that overlap in time on
    one GPU share the array and race."""
    torch = _torch()
    _check_prepared(prep)
    _need(w.codes, torch.uint8, "w.codes", 3)
    _need(w.scales, torch.uint8, "w.scales", 3)
    T, K = prep.bb_codes.shape[1], prep.K
    O = w.codes.shape[1]
    if w.K != K:
        raise ValueError("weight K does not match the activation K")
    _check_stage_major(w.codes, w.scales, O, K, "w")
    _check_matrix(out, torch.float32, T, O, "out")
    st = _lib.call("sharq_linear_scratchfree", prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(),
                   prep.res_codes.data_ptr(), prep.res_scales.data_ptr(), w.codes.data_ptr(), w.scales.data_ptr(),
                   T, O, K, out.data_ptr(), out.stride(0), _stream(out.device))
    _lib.check("sharq_linear_scratchfree", st)
    return out


def linear_grouped(prep: Prepared, w: MXFP4, seg_offsets, a_rows=None, out=None):
    """Grouped two-path GEMM over expert segments. w.codes is [E, G, O, 64];
    seg_offsets int32 [E+1]; a_rows int32 [P] (source row of each sorted pair) or None."""
    torch = _torch()
    _check_prepared(prep)
    _need(w.codes, torch.uint8, "w.codes", 4)
    _need(w.scales, torch.uint8, "w.scales", 4)
    _need(seg_offsets, torch.int32, "seg_offsets", 1)
    E, _, O, _ = w.codes.shape
    K = prep.K
    if w.K != K:
        raise ValueError("weight K does not match the activation K")
    _check_stage_major(w.codes[0], w.scales[0], O, K, "w")
    if seg_offsets.numel() != E + 1:
        raise ValueError("seg_offsets must have E + 1 entries")
    if a_rows is not None:
        _need(a_rows, torch.int32, "a_rows", 1)
        P = a_rows.numel()
    else:
        P = prep.bb_codes.shape[1]
    if out is None:
        out = torch.empty((P, O), dtype=torch.float32, device=w.codes.device)
    _check_matrix(out, torch.float32, P, O, "out", contiguous=True)
    st = _lib.call("sharq_linear_grouped", prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(),
                   prep.res_codes.data_ptr(), prep.res_scales.data_ptr(), prep.bb_codes.shape[1], _ptr(a_rows),
                   seg_offsets.data_ptr(), E, w.codes.data_ptr(), w.scales.data_ptr(), P, O, K, out.data_ptr(),
                   _stream(out.device))
    _lib.check("sharq_linear_grouped", st)
    return out


def linear_silu_prepare(prep: Prepared, w_gu: MXFP4, n: int = 2, m: int = 4, with_h: bool = False,
                        with_prepared: bool = True, with_mask: bool = True, split_k: bool = True):
    """Fused gate|up projection: Y = two-path GEMM of prep against w_gu (rows:
    I gate rows, then I up rows), h = bf16(silu(Y[:, :I]) * Y[:, I:]), then
    prepare(h, n, m). Returns (Prepared of h or None, h or None); the results
    equal linear(split_k) -> silu_mul -> prepare bit for bit. With split_k,
    problems with too few tiles to fill the GPU split K as linear does
    (sharq_linear_silu_prepare_ws over the cached workspace)."""
    torch = _torch()
    _check_prepared(prep)
    _need(w_gu.codes, torch.uint8, "w_gu.codes", 3)
    _need(w_gu.scales, torch.uint8, "w_gu.scales", 3)
    T, K = prep.bb_codes.shape[1], prep.K
    O = w_gu.codes.shape[1]
    if w_gu.K != K or O % 2:
        raise ValueError("w_gu must be [2I, K] with the activation's K")
    _check_stage_major(w_gu.codes, w_gu.scales, O, K, "w_gu")
    I = O // 2
    dev = prep.bb_codes.device
    kw = dict(dtype=torch.uint8, device=dev)
    h = torch.empty((T, I), dtype=torch.bfloat16, device=dev) if with_h else None
    hp = None
    if with_prepared:
        G = stages(I)
        hp = Prepared(torch.empty((G, T, 64), **kw), torch.empty((G, T, 4), **kw),
                      torch.empty((G, T, 64), **kw), torch.empty((G, T, 4), **kw),
                      torch.empty((T, I // 8), **kw) if with_mask else None, I)
    _fused_call(prep, w_gu, T, I, K, n, m, h, hp, split_k)
    return hp, h


def linear_silu_prepare_into(prep: Prepared, w_gu: MXFP4, out: Prepared, n: int = 2, m: int = 4,
                             split_k: bool = True) -> Prepared:
    """linear_silu_prepare writing prepare(h) into preallocated `out` (no h)."""
    _check_prepared(prep)
    _check_prepared(out)
    T, K, I = prep.bb_codes.shape[1], prep.K, out.K
    if w_gu.K != K or tuple(w_gu.codes.shape) != (stages(K), 2 * I, 64) or out.bb_codes.shape[1] != T:
        raise ValueError("shapes of prep, w_gu and out do not match")
    _fused_call(prep, w_gu, T, I, K, n, m, None, out, split_k)
    return out


def _fused_call(prep, w_gu, T, I, K, n, m, h, hp, split_k):
    dev = prep.bb_codes.device
    args = (prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(), prep.res_codes.data_ptr(),
            prep.res_scales.data_ptr(), w_gu.codes.data_ptr(), w_gu.scales.data_ptr(), T, I, K, n, m, _ptr(h),
            _ptr(hp and hp.bb_codes), _ptr(hp and hp.bb_scales), _ptr(hp and hp.res_codes),
            _ptr(hp and hp.res_scales), _ptr(hp and hp.mask))
    nbytes = _lib.call("sharq_linear_silu_prepare_workspace_bytes", T, I, K) if split_k else 0
    if nbytes > 0:
        ws = _workspace(dev, nbytes)
        st = _lib.call("sharq_linear_silu_prepare_ws", *args, ws.data_ptr(), ws.numel(), _stream(dev))
        _lib.check("sharq_linear_silu_prepare_ws", st)
        return
    st = _lib.call("sharq_linear_silu_prepare", *args, _stream(dev))
    _lib.check("sharq_linear_silu_prepare", st)


def linear_grouped_silu_prepare(prep: Prepared, w_gu: MXFP4, seg_offsets, a_rows=None, n: int = 2, m: int = 4,
                                with_h: bool = False, with_prepared: bool = True, with_mask: bool = True,
                                out: Prepared = None):
    """Grouped fused gate|up projection: linear_grouped against each expert's
    w_gu ([E, G, 2I, 64]: I gate rows, then I up rows), then silu_mul and
    prepare(h, n, m), in one kernel. Rows are the sorted pairs. Returns
    (Prepared of h or None, h or None), bit-identical to the three-step chain.
    `out` (a Prepared of [G_I, P, ...]) receives prepare(h) when given."""
    torch = _torch()
    _check_prepared(prep)
    _need(w_gu.codes, torch.uint8, "w_gu.codes", 4)
    _need(w_gu.scales, torch.uint8, "w_gu.scales", 4)
    _need(seg_offsets, torch.int32, "seg_offsets", 1)
    E, _, O, _ = w_gu.codes.shape
    K = prep.K
    if w_gu.K != K or O % 2:
        raise ValueError("w_gu must be [E, 2I, K] with the activation's K")
    _check_stage_major(w_gu.codes[0], w_gu.scales[0], O, K, "w_gu")
    if seg_offsets.numel() != E + 1:
        raise ValueError("seg_offsets must have E + 1 entries")
    if a_rows is not None:
        _need(a_rows, torch.int32, "a_rows", 1)
        P = a_rows.numel()
    else:
        P = prep.bb_codes.shape[1]
    I = O // 2
    dev = prep.bb_codes.device
    kw = dict(dtype=torch.uint8, device=dev)
    h = torch.empty((P, I), dtype=torch.bfloat16, device=dev) if with_h else None
    hp = None
    if out is not None:
        _check_prepared(out)
        if out.K != I or out.bb_codes.shape[1] != P:
            raise ValueError("out must be a Prepared of [P, I]")
        hp = out
    elif with_prepared:
        G = stages(I)
        hp = Prepared(torch.empty((G, P, 64), **kw), torch.empty((G, P, 4), **kw),
                      torch.empty((G, P, 64), **kw), torch.empty((G, P, 4), **kw),
                      torch.empty((P, I // 8), **kw) if with_mask else None, I)
    st = _lib.call("sharq_linear_grouped_silu_prepare", prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(),
                   prep.res_codes.data_ptr(), prep.res_scales.data_ptr(), prep.bb_codes.shape[1], _ptr(a_rows),
                   seg_offsets.data_ptr(), E, w_gu.codes.data_ptr(), w_gu.scales.data_ptr(), P, I, K, n, m, _ptr(h),
                   _ptr(hp and hp.bb_codes), _ptr(hp and hp.bb_scales), _ptr(hp and hp.res_codes),
                   _ptr(hp and hp.res_scales), _ptr(hp and hp.mask), _stream(dev))
    _lib.check("sharq_linear_grouped_silu_prepare", st)
    return hp, h


class CompactBackbone(NamedTuple):
    """A compressed backbone: kept codes [T, K/4] (row-major), per-group rank
    fields [T, meta_row_bytes], the n:m pattern and K. The backbone's block
    scales stay in the Prepared it came from."""
    codes: "object"
    meta: "object"
    n: int
    m: int
    K: int


def compress_backbone(prep: Prepared, n: int = 2, m: int = 4, out: CompactBackbone = None) -> CompactBackbone:
    """The compressed form of prep's backbone (needs prep.mask)."""
    torch = _torch()
    _check_prepared(prep)
    if prep.mask is None:
        raise ValueError("compressing the backbone needs the mask")
    T, K = prep.bb_codes.shape[1], prep.K
    row = _lib.call("sharq_backbone_meta_row_bytes", K, n, m)
    _lib.check("sharq_backbone_meta_row_bytes", int(min(row, 0)))
    if out is None:
        dev = prep.bb_codes.device
        out = CompactBackbone(torch.empty((T, K // 4), dtype=torch.uint8, device=dev),
                              torch.empty((T, row), dtype=torch.uint8, device=dev), n, m, K)
    if tuple(out.codes.shape) != (T, K // 4) or tuple(out.meta.shape) != (T, row) or (out.n, out.m, out.K) != (n, m, K):
        raise ValueError("out does not match the backbone")
    st = _lib.call("sharq_compress_backbone", prep.bb_codes.data_ptr(), prep.mask.data_ptr(), T, K, n, m,
                   out.codes.data_ptr(), out.meta.data_ptr(), _stream(prep.bb_codes.device))
    _lib.check("sharq_compress_backbone", st)
    return out


def expand_backbone(cb: CompactBackbone, bb_codes=None, mask=None, with_mask: bool = True):
    """Dense stage-major backbone codes [G, T, 64] (and the mask [T, K/8])
    from a CompactBackbone. Returns (bb_codes, mask or None)."""
    torch = _torch()
    _need(cb.codes, torch.uint8, "codes", 2)
    _need(cb.meta, torch.uint8, "meta", 2)
    T, K = cb.codes.shape[0], cb.K
    dev = cb.codes.device
    if bb_codes is None:
        bb_codes = torch.empty((stages(K), T, 64), dtype=torch.uint8, device=dev)
    if with_mask and mask is None:
        mask = torch.empty((T, K // 8), dtype=torch.uint8, device=dev)
    if not with_mask:
        mask = None
    _need(bb_codes, torch.uint8, "bb_codes", 3)
    if tuple(bb_codes.shape) != (stages(K), T, 64) or not bb_codes.is_contiguous():
        raise ValueError(f"bb_codes must be a contiguous [{stages(K)}, {T}, 64] tensor")
    if mask is not None:
        _check_matrix(mask, torch.uint8, T, K // 8, "mask", contiguous=True)
    st = _lib.call("sharq_expand_backbone", cb.codes.data_ptr(), cb.meta.data_ptr(), T, K, cb.n, cb.m,
                   bb_codes.data_ptr(), _ptr(mask), _stream(dev))
    _lib.check("sharq_expand_backbone", st)
    return bb_codes, mask


def moe_combine(y, pair_index, weights, out=None, bf16: bool = False):
    """out[t] = sum_j weights[t, j] * y[pair_index[t, j]] (slots with -1 skipped),
    fp32 accumulation in slot order; fp32 [T, H] or, with bf16, bf16 [T, H]."""
    torch = _torch()
    _need(y, torch.float32, "y", 2)
    _need(pair_index, torch.int32, "pair_index", 2)
    _need(weights, torch.float32, "weights", 2)
    if not (y.is_contiguous() and pair_index.is_contiguous() and weights.is_contiguous()):
        raise ValueError("y, pair_index and weights must be contiguous")
    if pair_index.shape != weights.shape:
        raise ValueError("pair_index and weights must have the same [T, k] shape")
    T, k = pair_index.shape
    P, H = y.shape
    dt = torch.bfloat16 if bf16 else torch.float32
    if out is None:
        out = torch.empty((T, H), dtype=dt, device=y.device)
    _check_matrix(out, dt, T, H, "out", contiguous=True)
    st = _lib.call("sharq_moe_combine", y.data_ptr(), P, H, pair_index.data_ptr(), weights.data_ptr(), T, k,
                   0 if bf16 else out.data_ptr(), out.data_ptr() if bf16 else 0, _stream(y.device))
    _lib.check("sharq_moe_combine", st)
    return out


def silu_mul(gu, out=None):
    """h = bf16(silu(gu[:, :I]) * gu[:, I:]) for a fused gate|up output gu fp32 [T, 2I]."""
    torch = _torch()
    _need(gu, torch.float32, "gu", 2)
    if not gu.is_contiguous():
        raise ValueError("gu must be contiguous")
    T, I2 = gu.shape
    I = I2 // 2
    if out is None:
        out = torch.empty((T, I), dtype=torch.bfloat16, device=gu.device)
    _check_matrix(out, torch.bfloat16, T, I, "out", contiguous=True)
    st = _lib.call("sharq_silu_mul", gu.data_ptr(), T, I, out.data_ptr(), _stream(gu.device))
    _lib.check("sharq_silu_mul", st)
    return out


# ---------------------------------------------------------------------------
# NVFP4: 16-entry E2M1 blocks with E4M3 block scales and an fp32 tensor scale
# ---------------------------------------------------------------------------


class NVPrepared(NamedTuple):
    """Outputs of the NVFP4 prepare: codes [G, T, 64] as in Prepared, E4M3
    block scales [G, T, 8] (byte j of a row's stage g covers K entries
    128 g + 16 j .. + 15), the mask, K and the activation's tensor scale."""
    bb_codes: "object"
    bb_scales: "object"
    res_codes: "object"
    res_scales: "object"
    mask: "object"
    K: int
    tensor_scale: float


class NVFP4(NamedTuple):
    """An NVFP4 tensor, stage-major: codes [G, R, 64], E4M3 scales [G, R, 8]."""
    codes: "object"
    scales: "object"
    K: int
    tensor_scale: float


def _check_nv(codes, scales, R, K, name):
    torch = _torch()
    _need(codes, torch.uint8, name + ".codes", 3)
    _need(scales, torch.uint8, name + ".scales", 3)
    G = stages(K)
    if tuple(codes.shape) != (G, R, 64) or tuple(scales.shape) != (G, R, 8):
        raise ValueError(f"{name}: expected codes [{G}, {R}, 64] and scales [{G}, {R}, 8], "
                         f"got {tuple(codes.shape)} and {tuple(scales.shape)}")
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError(f"{name}: codes and scales must be contiguous")


def prepare_nvfp4(x, tensor_scale: float, gamma=None, n: int = 2, m: int = 4, with_mask: bool = True,
                  out: Optional[NVPrepared] = None) -> NVPrepared:
    """The prepare operator with NVFP4 codes; tensor_scale is the activation's
    fp32 tensor scale (shared by backbone and residual)."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous along K")
    T, K = x.shape
    if gamma is not None:
        _need(gamma, torch.bfloat16, "gamma", 1)
        if gamma.numel() != K:  # the kernels read K entries of gamma
            raise ValueError(f"gamma must hold K = {K} entries, got {gamma.numel()}")
        gamma = gamma.contiguous()
    if out is None:
        kw = dict(dtype=torch.uint8, device=x.device)
        G = stages(K)
        out = NVPrepared(torch.empty((G, T, 64), **kw), torch.empty((G, T, 8), **kw),
                         torch.empty((G, T, 64), **kw), torch.empty((G, T, 8), **kw),
                         torch.empty((T, K // 8), **kw) if with_mask else None, K, float(tensor_scale))
    else:
        if out.K != K:
            raise ValueError("out was allocated for another K")
        _check_nv(out.bb_codes, out.bb_scales, T, K, "out backbone")
        _check_nv(out.res_codes, out.res_scales, T, K, "out residual")
        if out.mask is not None:
            _check_matrix(out.mask, torch.uint8, T, K // 8, "out.mask", contiguous=True)
        out = out._replace(tensor_scale=float(tensor_scale))
    st = _lib.call("sharq_prepare_nvfp4", x.data_ptr(), T, K, x.stride(0), _ptr(gamma), n, m, float(tensor_scale),
                   out.bb_codes.data_ptr(), out.bb_scales.data_ptr(), out.res_codes.data_ptr(),
                   out.res_scales.data_ptr(), _ptr(out.mask), _stream(x.device))
    _lib.check("sharq_prepare_nvfp4", st)
    return out


def quantize_nvfp4(w, tensor_scale: float, out: Optional[NVFP4] = None) -> NVFP4:
    """NVFP4 of a bf16 [O, K] tensor with the given fp32 tensor scale."""
    torch = _torch()
    _need(w, torch.bfloat16, "w", 2)
    if w.stride(1) != 1:
        raise ValueError("w rows must be contiguous along K")
    O, K = w.shape
    if out is None:
        out = NVFP4(torch.empty((stages(K), O, 64), dtype=torch.uint8, device=w.device),
                    torch.empty((stages(K), O, 8), dtype=torch.uint8, device=w.device), K, float(tensor_scale))
    else:
        _check_nv(out.codes, out.scales, O, K, "out")
        out = out._replace(tensor_scale=float(tensor_scale))
    st = _lib.call("sharq_quantize_nvfp4", w.data_ptr(), O, K, w.stride(0), float(tensor_scale),
                   out.codes.data_ptr(), out.scales.data_ptr(), _stream(w.device))
    _lib.check("sharq_quantize_nvfp4", st)
    return out


def linear_nvfp4(prep: NVPrepared, w: NVFP4, out=None):
    """Two-path GEMM on NVFP4 operands: Y = deq(A_s) W^T + deq(A_r) W^T, fp32 [T, O]."""
    torch = _torch()
    T, K = prep.bb_codes.shape[1], prep.K
    O = w.codes.shape[1]
    _check_nv(prep.bb_codes, prep.bb_scales, T, K, "backbone")
    _check_nv(prep.res_codes, prep.res_scales, T, K, "residual")
    _check_nv(w.codes, w.scales, O, K, "w")
    if w.K != K:
        raise ValueError("weight K does not match the activation K")
    if out is None:
        out = torch.empty((T, O), dtype=torch.float32, device=prep.bb_codes.device)
    _check_matrix(out, torch.float32, T, O, "out")
    st = _lib.call("sharq_linear_nvfp4", prep.bb_codes.data_ptr(), prep.bb_scales.data_ptr(),
                   prep.res_codes.data_ptr(), prep.res_scales.data_ptr(), float(prep.tensor_scale),
                   w.codes.data_ptr(), w.scales.data_ptr(), float(w.tensor_scale), T, O, K, out.data_ptr(),
                   out.stride(0), _stream(out.device))
    _lib.check("sharq_linear_nvfp4", st)
    return out


# ---------------------------------------------------------------------------
# Layout conversion: canonical row-major block-FP4 <-> stage-major
# ---------------------------------------------------------------------------


def _pack(codes_rm, scales_rm, K, block, name):
    torch = _torch()
    _need(codes_rm, torch.uint8, name + " codes", 2)
    _need(scales_rm, torch.uint8, name + " scales", 2)
    R = codes_rm.shape[0]
    _check_matrix(codes_rm, torch.uint8, R, K // 2, name + " codes", contiguous=True)
    _check_matrix(scales_rm, torch.uint8, R, K // block, name + " scales", contiguous=True)
    G = stages(K)
    codes = torch.empty((G, R, 64), dtype=torch.uint8, device=codes_rm.device)
    scales = torch.empty((G, R, 128 // block), dtype=torch.uint8, device=codes_rm.device)
    st = _lib.call("sharq_pack_stage_major", codes_rm.data_ptr(), scales_rm.data_ptr(), R, K, block,
                   codes.data_ptr(), scales.data_ptr(), _stream(codes_rm.device))
    _lib.check("sharq_pack_stage_major", st)
    return codes, scales


def pack_mxfp4(codes_rm, scales_rm, K: int) -> MXFP4:
    """An MXFP4 tensor from the canonical row-major layout (codes [R, K/2],
    E8M0 scale bytes [R, K/32]), e.g. a weight quantised elsewhere."""
    codes, scales = _pack(codes_rm, scales_rm, K, 32, "MXFP4")
    return MXFP4(codes, scales, K)


def pack_nvfp4(codes_rm, scales_rm, K: int, tensor_scale: float) -> NVFP4:
    """An NVFP4 tensor from the canonical row-major layout (codes [R, K/2],
    E4M3 scale bytes [R, K/16]) and its fp32 tensor scale."""
    codes, scales = _pack(codes_rm, scales_rm, K, 16, "NVFP4")
    return NVFP4(codes, scales, K, float(tensor_scale))


def unpack_stage_major(codes, scales, K: int):
    """(codes [R, K/2], scales [R, K/block]) in the canonical row-major layout
    from stage-major codes [G, R, 64] and scales [G, R, 128/block] (block 32
    for MXFP4 scales [G, R, 4], 16 for NVFP4 scales [G, R, 8])."""
    torch = _torch()
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    G, R, _ = codes.shape
    per = scales.shape[2]
    if per not in (4, 8) or tuple(codes.shape) != (stages(K), R, 64) or tuple(scales.shape) != (stages(K), R, per) \
            or not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("expected contiguous stage-major codes [G, R, 64] and scales [G, R, 4 or 8]")
    block = 128 // per
    codes_rm = torch.empty((R, K // 2), dtype=torch.uint8, device=codes.device)
    scales_rm = torch.empty((R, K // block), dtype=torch.uint8, device=codes.device)
    st = _lib.call("sharq_unpack_stage_major", codes.data_ptr(), scales.data_ptr(), R, K, block,
                   codes_rm.data_ptr(), scales_rm.data_ptr(), _stream(codes.device))
    _lib.check("sharq_unpack_stage_major", st)
    return codes_rm, scales_rm
