"""Host-side checks of the C ABI library (no GPU needed, no compute launched).

The library must load, export every function ``include/blockint8.h``
declares, and reject every bad argument on the host before any HIP call, with
the documented status.  Calls here never pass a valid argument set, so no
kernel is ever launched (fake pointers are used only where the call is
rejected first).
"""
import ctypes
import os
import re

import pytest
import torch

import block_wise_int8_amd as bi8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockint8.h")

OK, NULL, SHAPE, BLOCK, ALIGN, HIP = 0, 1, 2, 3, 4, 5
P16 = 0x10000          # fake, 16-byte aligned "device" address (never dereferenced)
P_ODD = 0x10001


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(blockint8_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bi8.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"blockint8_status_string", "blockint8_last_error",
                          "blockint8_quant_act", "blockint8_gemm", "blockint8_gemm_ws",
                          "blockint8_gemm_workspace_size", "blockint8_moe_gemm", "blockint8_moe_gemm_ws",
                          "blockint8_moe_gemm_workspace_size",
                          "blockint8_linear", "blockint8_linear_noalloc", "blockint8_moe_route", "blockint8_quant_act_gather",
                          "blockint8_quant_weight", "blockint8_check_tp_partition",
                          "blockint8_silu_mul_quant", "blockint8_moe_gemm_silu_quant", "blockint8_moe_combine", "blockint8_gemm_select", "blockint8_moe_gemm_select",
                          "blockint8_gemm_variant", "blockint8_moe_gemm_variant"}
    for name in names:
        assert hasattr(lib, name), name
    # exported with C linkage (no mangling) in the shared object
    raw = ctypes.CDLL(bi8.lib_path())
    for name in names:
        getattr(raw, name)


def test_status_strings(lib):
    for code, name in [(OK, "BI8_OK"), (NULL, "BI8_ERR_NULL"), (SHAPE, "BI8_ERR_SHAPE"),
                       (BLOCK, "BI8_ERR_BLOCK"), (ALIGN, "BI8_ERR_ALIGN"), (HIP, "BI8_ERR_HIP")]:
        assert lib.blockint8_status_string(code).decode() == name
    assert lib.blockint8_status_string(99).decode() == "BI8_ERR_UNKNOWN"


def quant(lib, x=P16, M=4, K=256, ldx=256, bk=128, xq=P16, xs=P16):
    return lib.blockint8_quant_act(x, M, K, ldx, bk, xq, xs, None)


def gemm(lib, xq=P16, xs=P16, w=P16, ws=P16, bias=None, y=P16, M=4, N=256, K=256, bn=128, bk=128):
    return lib.blockint8_gemm(xq, xs, w, ws, bias, y, M, N, K, bn, bk, None)


def moe(lib, xq=P16, xs=P16, off=P16, w=P16, ws=P16, y=P16, R=4, N=256, K=256, E=2, bn=128, bk=128):
    return lib.blockint8_moe_gemm(xq, xs, off, w, ws, y, R, N, K, E, bn, bk, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(xq=None), NULL), (dict(xs=None), NULL),
    (dict(M=-1), SHAPE), (dict(K=0), SHAPE), (dict(K=-16), SHAPE), (dict(K=1 << 24, ldx=1 << 24), SHAPE),
    (dict(ldx=128), SHAPE),
    (dict(bk=64), BLOCK), (dict(bk=0), BLOCK), (dict(bk=-128), BLOCK),
    (dict(x=P_ODD), ALIGN),   # any K and any row stride are accepted; x needs 2-byte alignment
    (dict(xq=P16 + 8), ALIGN), (dict(xs=P16 + 2), ALIGN),
])
def test_quant_rejects(lib, kw, status):
    assert quant(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_quant_act")


def test_quant_empty_is_noop(lib):
    assert quant(lib, M=0, x=None, xq=None, xs=None) == OK
    assert lib.blockint8_last_error().decode() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(xq=None), NULL), (dict(xs=None), NULL), (dict(w=None), NULL), (dict(ws=None), NULL),
    (dict(y=None), NULL),
    (dict(M=-1), SHAPE), (dict(N=0), SHAPE), (dict(N=-5), SHAPE), (dict(K=0), SHAPE),
    (dict(M=1 << 31), SHAPE), (dict(K=1 << 24), SHAPE),
    (dict(bn=0), BLOCK), (dict(bk=-1), BLOCK), (dict(bn=64), BLOCK), (dict(bk=256), BLOCK),
    (dict(bn=1, bk=128), BLOCK), (dict(bn=1, bk=512), BLOCK),   # (1, K) only with block_k == K
    (dict(bn=1, bk=1 << 18, K=1 << 18), SHAPE),                    # per-channel int32 sums: K <= 2^17
    (dict(xq=P16 + 4), ALIGN), (dict(w=P16 + 8), ALIGN),
    (dict(xs=P16 + 1), ALIGN), (dict(ws=P16 + 3), ALIGN), (dict(y=P_ODD), ALIGN),
    (dict(bias=P_ODD), ALIGN),
])
def test_gemm_rejects(lib, kw, status):
    assert gemm(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_gemm")


def gemm_ws_call(lib, xq=P16, xs=P16, w=P16, ws=P16, bias=None, y=P16, M=4, N=256, K=256, bn=128, bk=128,
                 wsp=P16, nbytes=1 << 20):
    return lib.blockint8_gemm_ws(xq, xs, w, ws, bias, y, M, N, K, bn, bk, wsp, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(xq=None), NULL), (dict(y=None), NULL), (dict(M=-1), SHAPE), (dict(K=0), SHAPE),
    (dict(nbytes=-1), SHAPE), (dict(bn=64), BLOCK), (dict(xq=P16 + 4), ALIGN), (dict(wsp=P16 + 8), ALIGN),
    (dict(bias=P_ODD), ALIGN),
])
def test_gemm_ws_rejects(lib, kw, status):
    assert gemm_ws_call(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_gemm_ws")


def test_gemm_workspace_size_host_rule(lib):
    """Split K only for grids of at most one 128 x 64 tile per CU, outputs of at
    most 640k entries and >= 16 K blocks."""
    size = lib.blockint8_gemm_workspace_size
    assert size(64, 8192, 4096, 128, 128) == 4 * 4 * 64 * 8192   # 64 tiles, 32 K blocks: 4 splits
    assert size(4096, 4096, 4096, 128, 128) == 0      # a full grid: no split
    assert size(333, 5000, 4000, 128, 128) == 0       # the partials would cost more than they save
    assert size(8, 4096, 4096, 128, 128) == 0         # the skinny kernel
    assert size(64, 8192, 1024, 128, 128) == 0        # too few K blocks
    assert size(64, 8192, 4001, 128, 128) == 0        # K % 16 != 0
    assert size(64, 8192, 4096, 1, 4096) == 0         # per-channel
    assert size(0, 5000, 4096, 128, 128) == 0 and size(10, 10, -1, 128, 128) == 0
    assert gemm_ws_call(lib, M=0, xq=None, xs=None, w=None, ws=None, y=None, wsp=None) == OK


def test_gemm_empty_is_noop(lib):
    assert gemm(lib, M=0, xq=None, xs=None, w=None, ws=None, y=None) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(off=None), NULL), (dict(w=None), NULL), (dict(xq=None), NULL),
    (dict(E=0), SHAPE), (dict(E=-1), SHAPE), (dict(E=65537), SHAPE), (dict(R=-1), SHAPE),
    (dict(N=0), SHAPE),
    (dict(bn=64), BLOCK),
    (dict(K=100), ALIGN), (dict(off=P16 + 2), ALIGN), (dict(xq=P16 + 4), ALIGN),
])
def test_moe_rejects(lib, kw, status):
    assert moe(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_moe_gemm")


def moe_ws(lib, xq=P16, xs=P16, off=P16, w=P16, ws=P16, y=P16, R=4, N=256, K=256, E=2, bn=128, bk=128,
           wsp=None, nbytes=0):
    return lib.blockint8_moe_gemm_ws(xq, xs, off, w, ws, y, R, N, K, E, bn, bk, wsp, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(off=None), NULL), (dict(w=None), NULL), (dict(xq=None), NULL),
    (dict(E=0), SHAPE), (dict(E=65537), SHAPE), (dict(R=-1), SHAPE), (dict(N=0), SHAPE),
    (dict(nbytes=-1), SHAPE),
    (dict(bn=64), BLOCK),
    (dict(K=100), ALIGN), (dict(off=P16 + 2), ALIGN), (dict(wsp=P16 + 4, nbytes=1 << 25), ALIGN),
])
def test_moe_ws_rejects(lib, kw, status):
    assert moe_ws(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_moe_gemm_ws")


def test_moe_gemm_workspace_size_host_rule(lib):
    mib32 = 256 * 128 * 256 * 4
    assert bi8.moe_gemm_workspace_size(8192, 4096, 14336, 8) == mib32     # w2 of the MoE layer: 256 x 128
    assert bi8.moe_gemm_workspace_size(700, 1024, 384, 3) == mib32
    assert bi8.moe_gemm_workspace_size(8192, 28672, 4096, 8) == 0         # w13: the 256 x 256 kernel
    for bad in [(0, 4096, 4096, 8), (8192, 0, 4096, 8), (8192, 4096, 100, 8), (8192, 4096, 4096, 0)]:
        assert bi8.moe_gemm_workspace_size(*bad) == 0
    assert lib.blockint8_moe_gemm_workspace_size(8192, 4096, 14336, 8, 64, 128) == 0


def test_moe_empty_is_noop(lib):
    assert moe(lib, R=0, xq=None, xs=None, off=None, w=None, ws=None, y=None) == OK


def test_binding_has_no_cpu_path():
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        bi8.quant_act(x)
    xq = torch.zeros((4, 128), dtype=torch.int8)
    xs = torch.zeros((4, 1), dtype=torch.float32)
    w = torch.zeros((8, 128), dtype=torch.int8)
    ws = torch.zeros((1, 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="HIP device"):
        bi8.gemm(xq, xs, w, ws)
    with pytest.raises(ValueError, match="HIP device"):
        bi8.moe_gemm(xq, xs, torch.zeros(2, dtype=torch.int32), w[None], ws[None])


def test_scale_shape_helper():
    assert bi8.scale_shape(4096, 4096) == (32, 32)
    assert bi8.scale_shape(5000, 4000) == (40, 32)


def test_variant_ids_match_header():
    text = open(HEADER).read()
    ids = dict((k, int(v)) for k, v in re.findall(r"\b(BI8_GEMM_\w+)\s*=\s*(\d+)", text))
    assert ids == {"BI8_GEMM_AUTO": bi8.GEMM_AUTO, "BI8_GEMM_SKINNY": bi8.GEMM_SKINNY,
                   "BI8_GEMM_TILE_128X64": bi8.GEMM_TILE_128X64,
                   "BI8_GEMM_TILE_256X128": bi8.GEMM_TILE_256X128,
                   "BI8_GEMM_TILE_256X256": bi8.GEMM_TILE_256X256}


@pytest.mark.parametrize("M,N,K,variant", [
    (1, 4096, 4096, bi8.GEMM_SKINNY), (32, 100, 128, bi8.GEMM_SKINNY),
    (33, 4096, 4096, bi8.GEMM_SKINNY), (64, 4096, 4096, bi8.GEMM_SKINNY),
    # the skinny kernel's traffic grows with N * (16 + M): past a budget the
    # tiled kernel runs, also for few tokens
    (64, 8192, 4096, bi8.GEMM_TILE_128X64), (32, 8192, 4096, bi8.GEMM_TILE_128X64),
    (8, 28672, 4096, bi8.GEMM_TILE_128X64), (65, 100, 128, bi8.GEMM_TILE_128X64),
    (333, 5000, 4000, bi8.GEMM_TILE_128X64),
    (2048, 4096, 14336, bi8.GEMM_TILE_256X128), (4096, 4096, 4096, bi8.GEMM_TILE_256X256),
    (2048, 28672, 4096, bi8.GEMM_TILE_256X256), (8192, 8192, 1024, bi8.GEMM_TILE_256X256),
])
def test_gemm_select(lib, M, N, K, variant):
    """The shape-based choice (a host function: no launch)."""
    assert bi8.gemm_select(M, N, K) == variant


def test_moe_gemm_select(lib):
    assert bi8.moe_gemm_select(8192, 28672, 4096, 8) == bi8.GEMM_TILE_256X256
    assert bi8.moe_gemm_select(8192, 4096, 14336, 8) == bi8.GEMM_TILE_256X128   # 512 wide tiles: 2 rounds
    assert bi8.moe_gemm_select(16384, 4096, 14336, 8) == bi8.GEMM_TILE_256X256  # 1024: 4 rounds
    assert bi8.moe_gemm_select(512, 4096, 4096, 8) == bi8.GEMM_TILE_256X128


def gemm_v(lib, variant, M=4, xq=P16, **kw):
    a = dict(xs=P16, w=P16, ws=P16, bias=None, y=P16, N=256, K=256, bn=128, bk=128)
    a.update(kw)
    return lib.blockint8_gemm_variant(variant, xq, a["xs"], a["w"], a["ws"], a["bias"], a["y"], M,
                                      a["N"], a["K"], a["bn"], a["bk"], None)


@pytest.mark.parametrize("variant,M,kw,status", [
    (-1, 4, {}, SHAPE), (5, 4, {}, SHAPE), (99, 4, {}, SHAPE),
    (bi8.GEMM_SKINNY, 65, {}, SHAPE),                       # skinny takes M <= 64
    (bi8.GEMM_TILE_256X256, 64, dict(xq=None), NULL),
    (bi8.GEMM_TILE_256X128, 64, dict(bk=64), BLOCK),
    (bi8.GEMM_TILE_128X64, 64, dict(K=72), ALIGN),          # K % 16 != 0: only AUTO
    (bi8.GEMM_SKINNY, 8, dict(K=4001), ALIGN),
    (bi8.GEMM_TILE_256X256, 300, dict(K=17), ALIGN),
])
def test_gemm_variant_rejects(lib, variant, M, kw, status):
    assert gemm_v(lib, variant, M=M, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_gemm")


def test_gemm_variant_empty_is_noop(lib):
    for v in range(5):
        assert gemm_v(lib, v, M=0, xq=None, xs=None, w=None, ws=None, y=None) == OK


@pytest.mark.parametrize("variant,status", [
    (bi8.GEMM_SKINNY, SHAPE), (bi8.GEMM_TILE_128X64, SHAPE), (7, SHAPE), (-2, SHAPE),
])
def test_moe_gemm_variant_rejects(lib, variant, status):
    assert lib.blockint8_moe_gemm_variant(variant, P16, P16, P16, P16, P16, P16, 4, 256, 256, 2, 128,
                                          128, None) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_moe_gemm")


def linear(lib, x=P16, ldx=256, w=P16, ws=P16, bias=None, y=P16, M=4, N=256, K=256, bn=128, bk=128,
           xq=P16, xs=P16):
    return lib.blockint8_linear(x, ldx, w, ws, bias, y, M, N, K, bn, bk, xq, xs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(ws=None), NULL), (dict(y=None), NULL),
    (dict(xq=None), NULL), (dict(xs=None), NULL),
    (dict(M=-1), SHAPE), (dict(N=0), SHAPE), (dict(K=0), SHAPE), (dict(ldx=128), SHAPE),
    (dict(bk=64), BLOCK), (dict(bn=256), BLOCK),
    (dict(x=P_ODD), ALIGN),
    (dict(w=P16 + 1), ALIGN), (dict(ws=P16 + 2), ALIGN), (dict(y=P_ODD), ALIGN), (dict(bias=P_ODD), ALIGN),
    (dict(xq=P16 + 4), ALIGN), (dict(xs=P16 + 1), ALIGN),
])
def test_linear_rejects(lib, kw, status):
    assert linear(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_linear")


def test_linear_empty_is_noop(lib):
    assert linear(lib, M=0, x=None, w=None, ws=None, y=None, xq=None, xs=None) == OK


def linear_noalloc(lib, x=P16, ldx=256, w=P16, ws=P16, bias=None, y=P16, M=4, N=256, K=256, bn=128, bk=128):
    return lib.blockint8_linear_noalloc(x, ldx, w, ws, bias, y, M, N, K, bn, bk, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(ws=None), NULL), (dict(y=None), NULL),
    (dict(M=-1), SHAPE), (dict(N=0), SHAPE), (dict(K=0), SHAPE), (dict(ldx=128), SHAPE),
    (dict(bk=64), BLOCK), (dict(bn=256), BLOCK),
    (dict(x=P_ODD), ALIGN),
    (dict(w=P16 + 1), ALIGN), (dict(ws=P16 + 2), ALIGN), (dict(y=P_ODD), ALIGN), (dict(bias=P_ODD), ALIGN),
])
def test_linear_noalloc_rejects(lib, kw, status):
    assert linear_noalloc(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_linear_noalloc")


def test_linear_noalloc_rejects_problems_larger_than_its_workspace(lib):
    # K = 4096: codes M * 4096 bytes + scales M * 32 * 4 bytes <= 20 MiB up to M = 4964
    assert (4964 * 4096 + 4 * 4964 * 32) <= bi8.NOALLOC_SCRATCH_BYTES < 4965 * 4096 + 4 * 4965 * 32
    assert linear_noalloc(lib, M=4965, K=4096, ldx=4096) == SHAPE
    msg = lib.blockint8_last_error().decode()
    assert "workspace" in msg and str(bi8.NOALLOC_SCRATCH_BYTES) in msg
    # per-channel form: one scale per row
    assert linear_noalloc(lib, M=(20 << 20) // 1024, K=1024, ldx=1024, bn=1, bk=1024) == SHAPE


def test_linear_noalloc_empty_is_noop(lib):
    assert linear_noalloc(lib, M=0, x=None, w=None, ws=None, y=None) == OK


def route(lib, logits=P16, T=16, E=8, k=2, ids=P16, w=P16, st=P16, off=P16, ro=P16):
    return lib.blockint8_moe_route(logits, T, E, k, 0, ids, w, st, off, ro, None)


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), NULL), (dict(ids=None), NULL), (dict(off=None), NULL), (dict(ro=None), NULL),
    (dict(E=0), SHAPE), (dict(E=1025), SHAPE), (dict(k=0), SHAPE), (dict(k=9, E=16), SHAPE),
    (dict(k=3, E=2), SHAPE), (dict(T=-1), SHAPE),
    (dict(logits=P16 + 2), ALIGN), (dict(off=P16 + 1), ALIGN), (dict(w=P16 + 3), ALIGN),
])
def test_moe_route_rejects(lib, kw, status):
    assert route(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_moe_route")


def gather(lib, x=P16, T=8, ldx=256, rows=P16, R=4, K=256, bk=128, xq=P16, xs=P16):
    return lib.blockint8_quant_act_gather(x, T, ldx, rows, R, K, bk, xq, xs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(rows=None), NULL), (dict(x=None), NULL), (dict(xq=None), NULL),
    (dict(R=-1), SHAPE), (dict(T=-1), SHAPE), (dict(K=0), SHAPE), (dict(ldx=128), SHAPE),
    (dict(bk=64), BLOCK), (dict(rows=P16 + 2), ALIGN), (dict(x=P_ODD), ALIGN),
])
def test_quant_act_gather_rejects(lib, kw, status):
    assert gather(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_quant_act_gather")


def silu(lib, h=P16, R=4, I=256, bk=128, aq=P16, as_=P16, a=None):
    return lib.blockint8_silu_mul_quant(h, R, I, bk, aq, as_, a, None)


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), NULL), (dict(aq=None), NULL), (dict(as_=None), NULL),
    (dict(R=-1), SHAPE), (dict(I=0), SHAPE), (dict(bk=256), BLOCK),
    (dict(I=40), ALIGN), (dict(h=P16 + 8), ALIGN), (dict(a=P16 + 8), ALIGN), (dict(as_=P16 + 2), ALIGN),
])
def test_silu_mul_quant_rejects(lib, kw, status):
    assert silu(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_silu_mul_quant")


def moe_silu(lib, xq=P16, xs=P16, off=P16, w=P16, ws=P16, aq=P16, as_=P16, R=4, I=256, K=256, E=2, bn=128,
             bk=128):
    return lib.blockint8_moe_gemm_silu_quant(xq, xs, off, w, ws, aq, as_, R, I, K, E, bn, bk, None)


@pytest.mark.parametrize("kw,status", [
    (dict(off=None), NULL), (dict(w=None), NULL), (dict(xq=None), NULL), (dict(aq=None), NULL),
    (dict(as_=None), NULL),
    (dict(E=0), SHAPE), (dict(E=65537), SHAPE), (dict(R=-1), SHAPE), (dict(I=0), SHAPE), (dict(I=-128), SHAPE),
    (dict(I=192), SHAPE), (dict(I=64), SHAPE),   # the fused epilogue takes whole 128-column groups
    (dict(bn=64), BLOCK), (dict(bk=256), BLOCK),
    (dict(K=100), ALIGN), (dict(off=P16 + 2), ALIGN), (dict(xq=P16 + 4), ALIGN), (dict(aq=P16 + 4), ALIGN),
    (dict(as_=P16 + 2), ALIGN), (dict(ws=P16 + 2), ALIGN),
])
def test_moe_gemm_silu_quant_rejects(lib, kw, status):
    assert moe_silu(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_moe_gemm_silu_quant")


def test_moe_gemm_silu_quant_empty_is_noop(lib):
    assert moe_silu(lib, R=0, xq=None, xs=None, off=None, w=None, ws=None, aq=None, as_=None) == OK


def combine(lib, y2=P16, R=8, ro=P16, w=P16, T=4, k=2, H=64, out=P16):
    return lib.blockint8_moe_combine(y2, R, ro, w, T, k, H, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(y2=None), NULL), (dict(ro=None), NULL), (dict(w=None), NULL), (dict(out=None), NULL),
    (dict(T=-1), SHAPE), (dict(R=-1), SHAPE), (dict(H=0), SHAPE), (dict(k=0), SHAPE),
    (dict(H=60), ALIGN), (dict(y2=P16 + 8), ALIGN), (dict(out=P16 + 4), ALIGN), (dict(ro=P16 + 1), ALIGN),
])
def test_moe_combine_rejects(lib, kw, status):
    assert combine(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_moe_combine")


def test_moe_steps_empty_are_noops(lib):
    assert gather(lib, R=0, x=None, rows=None, xq=None, xs=None) == OK
    assert silu(lib, R=0, h=None, aq=None, as_=None) == OK
    assert combine(lib, T=0, y2=None, ro=None, w=None, out=None) == OK


def tp_cases():
    path = os.path.join(ROOT, "tests", "golden", "tp_partition_cases.txt")
    for line in open(path):
        line = line.split("#")[0].split()
        if line:
            yield ([int(v) for v in line[:5]], [int(v) for v in line[5].split(",")], line[6])


@pytest.mark.parametrize("case", list(tp_cases()))
def test_check_tp_partition_follows_the_rule(lib, case):
    (ins, per, tp, bn, bk), outs, expected = case
    if expected == "ok":
        bi8.check_tp_partition(ins, per, outs, tp, block=(bn, bk))
        assert lib.blockint8_last_error().decode() == ""
    else:
        with pytest.raises(bi8.BlockInt8Error, match="BI8_ERR_BLOCK"):
            bi8.check_tp_partition(ins, per, outs, tp, block=(bn, bk))


def test_check_tp_partition_rejects_bad_arguments(lib):
    assert lib.blockint8_check_tp_partition(4096, 4096, None, 1, 1, 128, 128) == NULL
    assert lib.blockint8_check_tp_partition(0, 4096, None, 0, 1, 128, 128) == SHAPE
    assert lib.blockint8_check_tp_partition(4096, 4096, None, 0, 0, 128, 128) == SHAPE
    assert lib.blockint8_check_tp_partition(4096, 4096, None, 0, 1, 0, 128) == SHAPE
    with pytest.raises(bi8.BlockInt8Error, match="BI8_ERR_SHAPE"):
        bi8.check_tp_partition(4096, 4096, [128, 0], 1)


def qweight(lib, w=P16, N=256, K=256, ldw=256, bn=128, bk=128, wq=P16, ws=P16):
    return lib.blockint8_quant_weight(w, N, K, ldw, bn, bk, wq, ws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), NULL), (dict(wq=None), NULL), (dict(ws=None), NULL),
    (dict(N=-1), SHAPE), (dict(N=65536 * 128), SHAPE), (dict(K=0), SHAPE), (dict(ldw=128), SHAPE),
    (dict(bn=64), BLOCK), (dict(bk=256), BLOCK),
    (dict(K=200, ldw=200), ALIGN), (dict(ldw=260), ALIGN), (dict(w=P16 + 8), ALIGN), (dict(wq=P16 + 4), ALIGN),
    (dict(ws=P16 + 2), ALIGN),
])
def test_quant_weight_rejects(lib, kw, status):
    assert qweight(lib, **kw) == status
    assert lib.blockint8_last_error().decode().startswith("blockint8_quant_weight")


def test_quant_weight_empty_is_noop(lib):
    assert qweight(lib, N=0, w=None, wq=None, ws=None) == OK


def test_per_channel_blocks_are_checked_before_launch(lib):
    # the (1, K) form: variant must be AUTO, MoE does not take it
    assert gemm_v(lib, bi8.GEMM_TILE_256X128, M=64, bn=1, bk=256) == SHAPE
    assert gemm_v(lib, bi8.GEMM_AUTO, M=0, bn=1, bk=256, xq=None, xs=None, w=None, ws=None, y=None) == OK
    assert moe(lib, bn=1, bk=256) == BLOCK
    assert quant(lib, M=0, bk=256, x=None, xq=None, xs=None) == OK          # block_k == K: per token
    assert quant(lib, bk=64) == BLOCK
    assert linear(lib, bn=1, bk=1 << 18, K=1 << 18, ldx=1 << 18) == SHAPE
