"""The C-ABI library loads on the host, exports every entry point the header
declares, and rejects bad arguments before any HIP call (CPU only: no call
here reaches a kernel launch)."""

import os
import re
import subprocess

import pytest

from activation_sparsity_fp4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sharq.h")

A = 0x10000  # fake, 16-byte aligned device addresses: never dereferenced
B = 0x20000
C = 0x30000
D = 0x40000
E_ = 0x50000
F = 0x60000
G = 0x70000


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SHARQ_API[^;]*?\b(sharq_\w+)\s*\(", text, flags=re.S)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared_symbols()) == exported


def test_status_strings_and_version():
    assert _lib.call("sharq_abi_version") == 10
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert _lib.status_string(s)
    assert _lib.status_string(-99) == "unknown status"


def prep(x=A, T=4, K=64, ldx=64, gamma=0, n=2, m=4, bc=B, bs=C, rc=D, rs=E_, mask=F):
    return _lib.call("sharq_prepare", x, T, K, ldx, gamma, n, m, bc, bs, rc, rs, mask, 0)


def test_prepare_validation():
    assert prep(T=0) == _lib.SHARQ_OK  # no-op, no launch
    assert prep(x=0) == _lib.SHARQ_EINVAL
    assert prep(bc=0) == _lib.SHARQ_EINVAL
    assert prep(rs=0) == _lib.SHARQ_EINVAL
    assert prep(T=-1) == _lib.SHARQ_EINVAL
    assert prep(K=48, ldx=48) == _lib.SHARQ_EINVAL      # K % 32
    assert prep(K=0, ldx=0) == _lib.SHARQ_EINVAL
    assert prep(ldx=32) == _lib.SHARQ_EINVAL            # ldx < K
    assert prep(n=4, m=8) == _lib.SHARQ_EUNSUPPORTED
    assert prep(n=1, m=4) == _lib.SHARQ_EUNSUPPORTED
    assert prep(x=A + 2) == _lib.SHARQ_EALIGN
    assert prep(ldx=68) == _lib.SHARQ_EALIGN
    assert prep(gamma=G + 4) == _lib.SHARQ_EALIGN
    assert prep(mask=F + 8) == _lib.SHARQ_EALIGN
    assert prep(T=1 << 31) == _lib.SHARQ_EINVAL
    assert prep(T=1 << 26, K=1024, ldx=1024) == _lib.SHARQ_EINVAL  # too many blocks for 32-bit indexing


def test_prepare_k_multiple_of_m():
    # K = 96 is a multiple of 32 and of 16, so 8:16 accepts it (T = 0 keeps it a no-op)
    assert prep(n=8, m=16, K=96, ldx=96, T=0) == _lib.SHARQ_OK


def lin(T=4, O=8, K=64, y=G, ldy=8, **kw):
    args = dict(bc=A, bs=B, rc=C, rs=D, wc=E_, ws=F)
    args.update(kw)
    return _lib.call("sharq_linear", args["bc"], args["bs"], args["rc"], args["rs"], args["wc"], args["ws"],
                     T, O, K, y, ldy, 0)


def test_linear_validation():
    assert lin(T=0) == _lib.SHARQ_OK
    assert lin(O=0, ldy=0) == _lib.SHARQ_OK
    assert lin(y=0) == _lib.SHARQ_EINVAL
    assert lin(wc=0) == _lib.SHARQ_EINVAL
    assert lin(K=48) == _lib.SHARQ_EINVAL
    assert lin(ldy=4) == _lib.SHARQ_EINVAL
    assert lin(T=-3) == _lib.SHARQ_EINVAL
    assert lin(ws=F + 1) == _lib.SHARQ_EALIGN
    assert lin(y=G + 4) == _lib.SHARQ_EALIGN


def lin_sf(T=4, O=8, K=64, y=G, ldy=8, **kw):
    args = dict(bc=A, bs=B, rc=C, rs=D, wc=E_, ws=F)
    args.update(kw)
    return _lib.call("sharq_linear_scratchfree", args["bc"], args["bs"], args["rc"], args["rs"], args["wc"],
                     args["ws"], T, O, K, y, ldy, 0)


def test_linear_scratchfree_validation():
    """The scratch-free GEMM checks its arguments as sharq_linear does, and
    refuses, before any HIP call, a shape whose split-K partials exceed the
    static scratch array."""
    assert lin_sf(T=0) == _lib.SHARQ_OK
    assert lin_sf(y=0) == _lib.SHARQ_EINVAL
    assert lin_sf(K=48) == _lib.SHARQ_EINVAL
    assert lin_sf(ldy=4) == _lib.SHARQ_EINVAL
    assert lin_sf(ws=F + 1) == _lib.SHARQ_EALIGN
    T, O, K = 320, 8192, 28672
    assert _lib.call("sharq_linear_workspace_bytes", T, O, K) > _lib.SCRATCHFREE_MAX_BYTES
    assert lin_sf(T=T, O=O, K=K, ldy=O) == _lib.SHARQ_ESCRATCH
    assert _lib.status_string(_lib.SHARQ_ESCRATCH) != "unknown status"
    header = open(HEADER).read()
    assert re.search(r"#define SHARQ_SCRATCHFREE_MAX_BYTES \(\(int64_t\)32 << 20\)", header)


def grp(P=16, O=8, K=64, E=2, a_rows=A, seg=B, T_src=16, **kw):
    return _lib.call("sharq_linear_grouped", C, D, E_, F, T_src, a_rows, seg, E, G, G + 4096, P, O, K, 0x90000, 0)


def test_grouped_validation():
    assert grp(P=0) == _lib.SHARQ_OK
    assert grp(E=0) == _lib.SHARQ_EINVAL
    assert grp(seg=0) == _lib.SHARQ_EINVAL
    assert grp(K=40) == _lib.SHARQ_EINVAL
    assert grp(a_rows=A + 4) == _lib.SHARQ_EALIGN
    assert grp(P=1 << 24, E=1, O=1 << 16) == _lib.SHARQ_EINVAL  # grid bound: over 2^24 tiles
    assert grp(P=128, E=1 << 20, O=1 << 13) == _lib.SHARQ_EINVAL  # grid bound from the experts
    assert grp(a_rows=0, T_src=8) == _lib.SHARQ_EINVAL  # identity rows need T_src >= P
    assert grp(T_src=-1) == _lib.SHARQ_EINVAL


def test_silu_and_quantize_validation():
    assert _lib.call("sharq_silu_mul", A, 0, 16, B, 0) == _lib.SHARQ_OK
    assert _lib.call("sharq_silu_mul", A, 4, 12, B, 0) == _lib.SHARQ_EINVAL
    assert _lib.call("sharq_silu_mul", 0, 4, 16, B, 0) == _lib.SHARQ_EINVAL
    assert _lib.call("sharq_silu_mul", A + 4, 4, 16, B, 0) == _lib.SHARQ_EALIGN
    assert _lib.call("sharq_quantize_mxfp4", A, 0, 64, 64, B, C, 0) == _lib.SHARQ_OK
    assert _lib.call("sharq_quantize_mxfp4", A, 2, 64, 64, 0, C, 0) == _lib.SHARQ_EINVAL
    assert _lib.call("sharq_quantize_mxfp4", A, 2, 50, 64, B, C, 0) == _lib.SHARQ_EINVAL
    assert _lib.call("sharq_quantize_mxfp4", A, 2, 64, 64, B, C + 1, 0) == _lib.SHARQ_EALIGN


def test_python_wrappers_refuse_cpu_tensors():
    torch = pytest.importorskip("torch")
    import activation_sparsity_fp4_amd as sq
    with pytest.raises(ValueError):
        sq.prepare(torch.zeros((2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        sq.silu_mul(torch.zeros((2, 16), dtype=torch.float32))


def fused(T=4, I=128, K=128, n=2, m=4, h=G, hbc=A + 0x100000, hbs=B + 0x100000, hrc=C + 0x100000,
          hrs=D + 0x100000, hmask=0, **kw):
    args = dict(bc=A, bs=B, rc=C, rs=D, wc=E_, ws=F)
    args.update(kw)
    return _lib.call("sharq_linear_silu_prepare", args["bc"], args["bs"], args["rc"], args["rs"], args["wc"],
                     args["ws"], T, I, K, n, m, h, hbc, hbs, hrc, hrs, hmask, 0)


def test_linear_silu_prepare_validation():
    assert fused(T=0) == _lib.SHARQ_OK
    assert fused(T=0, h=0) == _lib.SHARQ_OK                   # prepared output only
    assert fused(T=0, hbc=0, hbs=0, hrc=0, hrs=0) == _lib.SHARQ_OK  # h only
    assert fused(hbc=0, hbs=0, hrc=0, hrs=0, h=0) == _lib.SHARQ_EINVAL  # nothing to write
    assert fused(hbs=0) == _lib.SHARQ_EINVAL                  # prepared output half given
    assert fused(hbc=0, hbs=0, hrc=0, hrs=0, hmask=A) == _lib.SHARQ_EINVAL  # mask without prepare
    assert fused(n=4, m=8) == _lib.SHARQ_EUNSUPPORTED
    assert fused(T=-1) == _lib.SHARQ_EINVAL
    assert fused(K=96) == _lib.SHARQ_ENOTIMPL                  # K % 128
    assert fused(I=96) == _lib.SHARQ_ENOTIMPL                  # I % 128
    assert fused(I=100) == _lib.SHARQ_EINVAL                   # I % 32
    assert fused(bc=0) == _lib.SHARQ_EINVAL
    assert fused(wc=E_ + 4) == _lib.SHARQ_EALIGN
    assert fused(h=G + 2) == _lib.SHARQ_EALIGN
    assert fused(hmask=F + 8) == _lib.SHARQ_EALIGN
    assert fused(T=1 << 20, K=1 << 12) == _lib.SHARQ_ENOTIMPL  # activation codes past 32-bit offsets


def test_linear_ws_validation():
    args = (A, B, C, D, E_, F)
    assert _lib.call("sharq_linear_ws", *args, 0, 8, 64, G, 8, 0, 0, 0) == _lib.SHARQ_OK      # T = 0
    assert _lib.call("sharq_linear_ws", *args, 4, 8, 48, G, 8, 0, 0, 0) == _lib.SHARQ_EINVAL  # K % 32
    assert _lib.call("sharq_linear_ws", *args, 4, 8, 64, G, 4, 0, 0, 0) == _lib.SHARQ_EINVAL  # ldy < O
    assert _lib.call("sharq_linear_ws", *args, 4, 8, 64, G, 8, 0, -1, 0) == _lib.SHARQ_EINVAL  # workspace bytes
    assert _lib.call("sharq_linear_ws", *args, 4, 8, 64, G, 8, A + 8, 1024, 0) == _lib.SHARQ_EALIGN
    assert _lib.call("sharq_linear_ws", A, B, C, D, E_, 0, 4, 8, 64, G, 8, 0, 0, 0) == _lib.SHARQ_EINVAL


def test_linear_workspace_bytes():
    ws = lambda T, O, K: _lib.call("sharq_linear_workspace_bytes", T, O, K)
    assert ws(2048, 28672, 4096) == 0        # enough tiles: no split
    assert ws(8, 4096, 96) == 0              # K % 128 != 0: no split
    assert ws(4, 8, 48) == 0                 # invalid shape
    assert ws(1, 57344, 8192) == 0           # a weight this wide streams at the HBM rate unsplit
    assert ws(1024, 4096, 4096) == 0         # short K: the partials would cost more than the idle CUs
    # decode down projection 8192 x 28672: 6 splits, partials [6][1][8192] fp32
    assert ws(1, 8192, 28672) == 6 * 1 * 8192 * 4
    # Llama-3.1-8B down projection at T = 384 (48 tiles for 256 CUs): 5 splits
    assert ws(384, 4096, 14336) == 5 * 384 * 4096 * 4
    # every plan: S whole partials, 2 <= S <= 16, each split over at least 4 stages
    for T in (1, 7, 32, 33, 64, 65, 130, 300, 777, 1024, 2048):
        for O, K in ((1000, 8192), (4096, 4096), (8192, 28672), (1024, 512), (57344, 8192), (256, 131072)):
            b = ws(T, O, K)
            if b:
                S = b // (T * O * 4)
                assert b == S * T * O * 4 and 2 <= S <= min(16, K // 128 // 4), (T, O, K, S)


def test_fused_workspace_bytes():
    ws = lambda T, O, K: _lib.call("sharq_linear_workspace_bytes", T, O, K)
    fw = lambda T, I, K: _lib.call("sharq_linear_silu_prepare_workspace_bytes", T, I, K)
    assert fw(0, 128, 128) == 0 and fw(-1, 128, 128) == 0
    assert fw(4, 96, 128) == 0 and fw(4, 128, 96) == 0   # I and K must be multiples of 128
    assert fw(2048, 14336, 4096) == 0                     # enough tiles: no split
    # the fused entry splits exactly as the plain GEMM over (T, 2 I, K)
    assert fw(1, 28672, 8192) == ws(1, 57344, 8192) == 0   # Llama-3.1-70B decode gate|up: whole
    for T, I, K in ((1, 1024, 4096), (5, 512, 2048), (64, 1024, 4096), (200, 512, 4096), (300, 512, 8192),
                    (1, 14336, 4096), (20, 14336, 4096), (50, 2048, 1024)):
        assert fw(T, I, K) == ws(T, 2 * I, K), (T, I, K)
    assert fw(200, 512, 4096) > 0


def prep_rms(x=A, T=4, K=64, ldx=64, gamma=0, eps=1e-5, n=2, m=4, rms=G, bc=B, bs=C, rc=D, rs=E_, mask=F):
    return _lib.call("sharq_prepare_rms", x, T, K, ldx, gamma, eps, n, m, rms, bc, bs, rc, rs, mask, 0)


def test_prepare_rms_validation():
    assert prep_rms(T=0) == _lib.SHARQ_OK
    assert prep_rms(rms=0) == _lib.SHARQ_EINVAL            # the scales are an output
    assert prep_rms(eps=0.0) == _lib.SHARQ_EINVAL
    assert prep_rms(eps=-1.0) == _lib.SHARQ_EINVAL
    assert prep_rms(eps=float("inf")) == _lib.SHARQ_EINVAL
    assert prep_rms(eps=float("nan")) == _lib.SHARQ_EINVAL
    assert prep_rms(n=4, m=8) == _lib.SHARQ_EUNSUPPORTED
    assert prep_rms(K=48, ldx=48) == _lib.SHARQ_EINVAL
    assert prep_rms(rms=G + 4) == _lib.SHARQ_EALIGN
    assert prep_rms(T=1, K=131104, ldx=131104) == _lib.SHARQ_ENOTIMPL  # more than 4096 blocks
    assert prep_rms(T=0, K=131072, ldx=131072) == _lib.SHARQ_OK


def gfused(P=4, I=128, K=128, n=2, m=4, h=G, hbc=A + 0x100000, hbs=B + 0x100000, hrc=C + 0x100000,
           hrs=D + 0x100000, hmask=0, E=2, T_src=8, a_rows=0, seg=A + 0x200000, **kw):
    args = dict(bc=A, bs=B, rc=C, rs=D, wc=E_, ws=F)
    args.update(kw)
    return _lib.call("sharq_linear_grouped_silu_prepare", args["bc"], args["bs"], args["rc"], args["rs"], T_src,
                     a_rows, seg, E, args["wc"], args["ws"], P, I, K, n, m, h, hbc, hbs, hrc, hrs, hmask, 0)


def test_linear_grouped_silu_prepare_validation():
    assert gfused(P=0) == _lib.SHARQ_OK
    assert gfused(P=0, h=0) == _lib.SHARQ_OK
    assert gfused(hbc=0, hbs=0, hrc=0, hrs=0, h=0) == _lib.SHARQ_EINVAL   # nothing to write
    assert gfused(hrs=0) == _lib.SHARQ_EINVAL                           # prepared output half given
    assert gfused(hbc=0, hbs=0, hrc=0, hrs=0, hmask=A) == _lib.SHARQ_EINVAL
    assert gfused(n=4, m=8) == _lib.SHARQ_EUNSUPPORTED
    assert gfused(E=0) == _lib.SHARQ_EINVAL
    assert gfused(seg=0) == _lib.SHARQ_EINVAL
    assert gfused(T_src=2) == _lib.SHARQ_EINVAL                         # identity rows need T_src >= P
    assert gfused(K=96) == _lib.SHARQ_ENOTIMPL
    assert gfused(I=96) == _lib.SHARQ_ENOTIMPL
    assert gfused(I=100) == _lib.SHARQ_EINVAL
    assert gfused(P=1 << 24, E=1, T_src=1 << 24, I=1 << 12) == _lib.SHARQ_EINVAL  # h block index bound
    assert gfused(P=128, E=1 << 20, I=1 << 12) == _lib.SHARQ_EINVAL      # grid bound: over 2^24 tiles
    assert gfused(a_rows=A + 4) == _lib.SHARQ_EALIGN
    assert gfused(h=G + 2) == _lib.SHARQ_EALIGN
    assert gfused(T_src=1 << 20, K=1 << 12, P=8) == _lib.SHARQ_ENOTIMPL  # activation codes past 32-bit offsets


def fused_ws(ws=A + 0x400000, nbytes=1 << 20, **kw):
    args = dict(T=4, I=128, K=128, n=2, m=4, h=G, hbc=A + 0x100000, hbs=B + 0x100000, hrc=C + 0x100000,
                hrs=D + 0x100000, hmask=0)
    args.update(kw)
    return _lib.call("sharq_linear_silu_prepare_ws", A, B, C, D, E_, F, args["T"], args["I"], args["K"], args["n"],
                     args["m"], args["h"], args["hbc"], args["hbs"], args["hrc"], args["hrs"], args["hmask"], ws,
                     nbytes, 0)


def test_linear_silu_prepare_ws_validation():
    assert fused_ws(T=0) == _lib.SHARQ_OK
    assert fused_ws(T=0, ws=0, nbytes=0) == _lib.SHARQ_OK
    assert fused_ws(n=4, m=8) == _lib.SHARQ_EUNSUPPORTED
    assert fused_ws(K=96) == _lib.SHARQ_ENOTIMPL
    assert fused_ws(hbs=0) == _lib.SHARQ_EINVAL
    assert fused_ws(nbytes=-1) == _lib.SHARQ_EINVAL
    assert fused_ws(ws=0, nbytes=16) == _lib.SHARQ_EINVAL
    assert fused_ws(ws=A + 0x400004) == _lib.SHARQ_EALIGN
    assert fused_ws(h=G + 2) == _lib.SHARQ_EALIGN


def test_compact_backbone_validation():
    assert _lib.call("sharq_backbone_meta_row_bytes", 4096, 2, 4) == 384
    assert _lib.call("sharq_backbone_meta_row_bytes", 14336, 8, 16) == 1568
    assert _lib.call("sharq_backbone_meta_row_bytes", 96, 2, 4) == _lib.SHARQ_ENOTIMPL
    assert _lib.call("sharq_backbone_meta_row_bytes", 100, 2, 4) == _lib.SHARQ_EINVAL
    assert _lib.call("sharq_backbone_meta_row_bytes", 128, 4, 8) == _lib.SHARQ_EUNSUPPORTED
    cmp = lambda *a: _lib.call("sharq_compress_backbone", *a)
    exp = lambda *a: _lib.call("sharq_expand_backbone", *a)
    assert cmp(A, B, 0, 128, 2, 4, C, D, 0) == _lib.SHARQ_OK
    assert cmp(A, B, 4, 96, 2, 4, C, D, 0) == _lib.SHARQ_ENOTIMPL
    assert cmp(A, 0, 4, 128, 2, 4, C, D, 0) == _lib.SHARQ_EINVAL      # the mask is required
    assert cmp(A, B, 4, 128, 8, 16, C + 4, D, 0) == _lib.SHARQ_EALIGN
    assert cmp(A, B, 4, 128, 3, 4, C, D, 0) == _lib.SHARQ_EUNSUPPORTED
    assert exp(A, 0, 4, 128, 2, 4, C, D, 0) == _lib.SHARQ_EINVAL
    assert exp(A, B, 4, 128, 2, 4, C, D + 2, 0) == _lib.SHARQ_EALIGN
    assert exp(A, B, -1, 128, 2, 4, C, D, 0) == _lib.SHARQ_EINVAL


def test_moe_combine_validation():
    call = lambda *a: _lib.call("sharq_moe_combine", *a)
    assert call(A, 8, 16, B, C, 0, 2, D, 0, 0) == _lib.SHARQ_OK
    assert call(A, 8, 18, B, C, 4, 2, D, 0, 0) == _lib.SHARQ_EINVAL       # H % 4
    assert call(A, 8, 16, B, C, 4, 0, D, 0, 0) == _lib.SHARQ_EINVAL       # k >= 1
    assert call(A, 8, 16, B, C, 4, 2, 0, 0, 0) == _lib.SHARQ_EINVAL       # no output
    assert call(A, 8, 16, 0, C, 4, 2, D, 0, 0) == _lib.SHARQ_EINVAL
    assert call(A + 4, 8, 16, B, C, 4, 2, D, 0, 0) == _lib.SHARQ_EALIGN
    assert call(A, 8, 16, B, C, 4, 2, 0, D + 4, 0) == _lib.SHARQ_EALIGN   # bf16 output needs 8 bytes
    assert call(A, 8, 16, B + 2, C, 4, 2, D, 0, 0) == _lib.SHARQ_EALIGN


def test_nvfp4_validation():
    prep = lambda T=4, K=64, ldx=64, s=1.0, n=2, m=4, x=A, bs=C: _lib.call(
        "sharq_prepare_nvfp4", x, T, K, ldx, 0, n, m, s, B, bs, D, E_, F, 0)
    assert prep(T=0) == _lib.SHARQ_OK
    assert prep(s=0.0) == _lib.SHARQ_EINVAL             # tensor scale must be > 0
    assert prep(s=-1.0) == _lib.SHARQ_EINVAL
    assert prep(s=float("inf")) == _lib.SHARQ_EINVAL
    assert prep(s=float("nan")) == _lib.SHARQ_EINVAL
    assert prep(K=48, ldx=48) == _lib.SHARQ_EINVAL      # K % 32
    assert prep(n=4, m=8) == _lib.SHARQ_EUNSUPPORTED
    assert prep(x=0) == _lib.SHARQ_EINVAL
    assert prep(bs=C + 8) == _lib.SHARQ_EALIGN
    q = lambda O=4, K=64, ldw=64, s=1.0, w=A: _lib.call("sharq_quantize_nvfp4", w, O, K, ldw, s, B, C, 0)
    assert q(O=0) == _lib.SHARQ_OK
    assert q(s=0.0) == _lib.SHARQ_EINVAL
    assert q(K=40, ldw=40) == _lib.SHARQ_EINVAL
    assert q(w=A + 2) == _lib.SHARQ_EALIGN
    lin = lambda T=4, O=8, K=64, ldy=8, sa=1.0, sw=1.0, y=G: _lib.call(
        "sharq_linear_nvfp4", A, B, C, D, sa, E_, F, sw, T, O, K, y, ldy, 0)
    assert lin(T=0) == _lib.SHARQ_OK
    assert lin(sa=0.0) == _lib.SHARQ_EINVAL
    assert lin(sw=float("inf")) == _lib.SHARQ_EINVAL
    assert lin(ldy=4) == _lib.SHARQ_EINVAL
    assert lin(K=48) == _lib.SHARQ_EINVAL
    assert lin(y=G + 4) == _lib.SHARQ_EALIGN
    assert lin(T=1 << 30, O=1 << 30) == _lib.SHARQ_EINVAL  # grid bound


def test_pack_validation():
    pk = lambda R=4, K=64, block=32, c=A, s=B, co=C, so=D: _lib.call(
        "sharq_pack_stage_major", c, s, R, K, block, co, so, 0)
    up = lambda R=4, K=64, block=32, c=A, s=B, co=C, so=D: _lib.call(
        "sharq_unpack_stage_major", c, s, R, K, block, co, so, 0)
    for f in (pk, up):
        assert f(R=0) == _lib.SHARQ_OK
        assert f(block=8) == _lib.SHARQ_EINVAL
        assert f(K=48) == _lib.SHARQ_EINVAL
        assert f(R=-1) == _lib.SHARQ_EINVAL
        assert f(c=0) == _lib.SHARQ_EINVAL
        assert f(c=A + 4) == _lib.SHARQ_EALIGN
        assert f(co=C + 8) == _lib.SHARQ_EALIGN
        assert f(R=1 << 24, K=1 << 12) == _lib.SHARQ_EINVAL  # stage-major bytes past 2^31
        assert f(s=B + 1, so=D + 3, R=0) == _lib.SHARQ_OK       # scale pointers may be unaligned
