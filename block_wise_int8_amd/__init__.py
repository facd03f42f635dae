"""Block-wise INT8 W8A8 linear for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libblockint8.so`` (declared in
``include/blockint8.h``).  It only marshals arguments: every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device
memory and streams.  There is no CPU fallback: if the library is missing or a
tensor is not on a HIP device, the call raises.

Entry points (same names as the C ABI, without the ``blockint8_`` prefix):

* :func:`quant_act`  -- bf16 [M, K] -> int8 [M, K] + fp32 [M, ceil(K/128)]
* :func:`gemm`       -- y = bf16(block-scaled int8 GEMM (+ bias)), [M, N]
* :func:`moe_gemm`   -- the same per expert over expert-sorted rows
* :func:`linear`     -- quant_act followed by gemm (the dynamic-scale linear)
* :func:`moe_route`, :func:`quant_act_gather`, :func:`silu_mul_quant`,
  :func:`moe_combine` -- the MoE steps around the grouped GEMM,
  :func:`moe_gemm_silu_quant` -- the w13 GEMM with the gating as its epilogue,
  and :func:`moe_layer`, the whole FusedMoE layer built from them

``gemm`` and ``moe_gemm`` pick a kernel by shape (:func:`gemm_select`,
:func:`moe_gemm_select`); their ``variant`` argument names one instead.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["BlockInt8Error", "lib_path", "load", "scale_shape", "quant_act", "gemm", "gemm_ws",
           "gemm_workspace_size", "moe_gemm", "moe_gemm_workspace_size",
           "linear", "linear_noalloc", "NOALLOC_SCRATCH_BYTES", "gemm_select", "moe_gemm_select", "moe_route", "quant_act_gather",
           "silu_mul_quant", "moe_gemm_silu_quant", "moe_combine", "moe_layer", "quant_weight", "check_tp_partition", "BLOCK", "GEMM_AUTO", "GEMM_SKINNY",
           "GEMM_TILE_128X64", "GEMM_TILE_256X128", "GEMM_TILE_256X256"]

BLOCK = 128
# size of the library's static workspace behind linear_noalloc (BI8_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 20 << 20
# kernel variant ids (BI8_GEMM_* in the C header)
GEMM_AUTO, GEMM_SKINNY, GEMM_TILE_128X64, GEMM_TILE_256X128, GEMM_TILE_256X256 = range(5)
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libblockint8.so"
_lib = None

BI8_OK = 0
_STATUS_NAMES = {0: "BI8_OK", 1: "BI8_ERR_NULL", 2: "BI8_ERR_SHAPE", 3: "BI8_ERR_BLOCK",
                 4: "BI8_ERR_ALIGN", 5: "BI8_ERR_HIP"}


class BlockInt8Error(RuntimeError):
    """A C ABI call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, str(status)), message))
        self.status = status


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load() -> ctypes.CDLL:
    """Load ``libblockint8.so`` (building it first if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.blockint8_status_string.argtypes = [i32]
    lib.blockint8_status_string.restype = ctypes.c_char_p
    lib.blockint8_last_error.argtypes = []
    lib.blockint8_last_error.restype = ctypes.c_char_p
    lib.blockint8_quant_act.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp]
    lib.blockint8_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.blockint8_moe_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.blockint8_gemm_ws.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, i64, vp]
    lib.blockint8_gemm_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    lib.blockint8_gemm_workspace_size.restype = i64
    lib.blockint8_gemm_select.argtypes = [i64, i64, i64]
    lib.blockint8_moe_gemm_select.argtypes = [i64, i64, i64, i32]
    lib.blockint8_gemm_variant.argtypes = [i32] + lib.blockint8_gemm.argtypes
    lib.blockint8_moe_gemm_variant.argtypes = [i32] + lib.blockint8_moe_gemm.argtypes
    lib.blockint8_moe_gemm_ws.argtypes = lib.blockint8_moe_gemm.argtypes[:-1] + [vp, i64, vp]
    lib.blockint8_moe_gemm_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.blockint8_moe_gemm_workspace_size.restype = i64
    lib.blockint8_linear.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp]
    lib.blockint8_linear_noalloc.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.blockint8_moe_route.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.blockint8_quant_weight.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, vp]
    lib.blockint8_check_tp_partition.argtypes = [i64, i64, vp, i32, i32, i32, i32]
    lib.blockint8_quant_act_gather.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, vp, vp]
    lib.blockint8_silu_mul_quant.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    lib.blockint8_moe_gemm_silu_quant.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.blockint8_moe_combine.argtypes = [vp, i64, vp, vp, i64, i32, i64, vp, vp]
    for f in ("blockint8_quant_act", "blockint8_gemm", "blockint8_gemm_ws", "blockint8_moe_gemm", "blockint8_linear",
              "blockint8_linear_noalloc",
              "blockint8_moe_route", "blockint8_quant_act_gather", "blockint8_quant_weight",
              "blockint8_check_tp_partition", "blockint8_silu_mul_quant", "blockint8_moe_gemm_silu_quant",
              "blockint8_moe_combine", "blockint8_gemm_select",
              "blockint8_moe_gemm_select", "blockint8_gemm_variant", "blockint8_moe_gemm_variant",
              "blockint8_moe_gemm_ws"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != BI8_OK:
        msg = load().blockint8_last_error().decode(errors="replace")
        raise BlockInt8Error(status, msg)


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device (got %s); there is no CPU path" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims (got shape %s)" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def scale_shape(N: int, K: int, block_n: int = BLOCK, block_k: int = BLOCK):
    """Shape of a block-scale tensor for an int8 [N, K] weight: ceil both dims."""
    return (N + block_n - 1) // block_n, (K + block_k - 1) // block_k


def quant_act(x: torch.Tensor, xq: torch.Tensor | None = None, xs: torch.Tensor | None = None,
              block_k: int = BLOCK):
    """Dynamic per-(token, 128-group) quantisation of bf16 ``x`` [M, K].

    Returns ``(xq int8 [M, K], xs float32 [M, ceil(K/128)])``.  ``x`` may have
    a row stride (leading dimension) larger than K.
    """
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.dtype != torch.bfloat16:
        raise TypeError("x must be a 2-D bfloat16 tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device; there is no CPU path")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    M, K = x.shape
    KB = (K + block_k - 1) // block_k
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((M, KB), dtype=torch.float32, device=x.device)
    _need(xq, "xq", torch.int8, 2)
    _need(xs, "xs", torch.float32, 2)
    if tuple(xq.shape) != (M, K) or tuple(xs.shape) != (M, KB):
        raise ValueError("output shapes must be [M, K] and [M, ceil(K/128)]")
    ldx = x.stride(0) if M > 1 else K
    _check(load().blockint8_quant_act(_ptr(x), M, K, ldx, block_k, _ptr(xq), _ptr(xs),
                                      _stream_handle(x.device)))
    return xq, xs


def gemm_select(M: int, N: int, K: int) -> int:
    """The kernel variant (``GEMM_*``) that ``gemm`` runs for this shape."""
    return int(load().blockint8_gemm_select(M, N, K))


def moe_gemm_select(R: int, N: int, K: int, E: int) -> int:
    """The kernel variant (``GEMM_*``) that ``moe_gemm`` runs for this shape."""
    return int(load().blockint8_moe_gemm_select(R, N, K, E))


def gemm(xq: torch.Tensor, xs: torch.Tensor, w: torch.Tensor, ws: torch.Tensor,
         bias: torch.Tensor | None = None, y: torch.Tensor | None = None,
         block=(BLOCK, BLOCK), variant: int | None = None) -> torch.Tensor:
    """Block-scaled int8 GEMM ``y = x . W^T`` -> bf16 [M, N].

    ``variant`` (one of ``GEMM_*``) runs a named kernel instead of the
    shape-based choice."""
    _need(xq, "xq", torch.int8, 2)
    _need(xs, "xs", torch.float32, 2)
    _need(w, "w", torch.int8, 2)
    _need(ws, "ws", torch.float32, 2)
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] with K = %d (got %s)" % (K, tuple(w.shape)))
    NB, KB = scale_shape(N, K, *block)
    if tuple(xs.shape) != (M, KB) or tuple(ws.shape) != (NB, KB):
        raise ValueError("scale shapes must be xs [M, %d] and ws [%d, %d]" % (KB, NB, KB))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must be [N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    args = (_ptr(xq), _ptr(xs), _ptr(w), _ptr(ws), _ptr(bias), _ptr(y), M, N, K, block[0], block[1],
            _stream_handle(xq.device))
    if variant is None:
        _check(load().blockint8_gemm(*args))
    else:
        _check(load().blockint8_gemm_variant(int(variant), *args))
    return y


def gemm_workspace_size(M: int, N: int, K: int, block=(BLOCK, BLOCK)) -> int:
    """Bytes of workspace ``gemm_ws`` uses for an M x N x K problem (0: none)."""
    return int(load().blockint8_gemm_workspace_size(M, N, K, block[0], block[1]))


def gemm_ws(xq: torch.Tensor, xs: torch.Tensor, w: torch.Tensor, ws: torch.Tensor,
            workspace: torch.Tensor | None, bias: torch.Tensor | None = None, y: torch.Tensor | None = None,
            block=(BLOCK, BLOCK)) -> torch.Tensor:
    """``gemm`` with a caller workspace (any dtype, contiguous, on the device; or
    None), which lets problems with few tiles split K between workgroups."""
    _need(xq, "xq", torch.int8, 2)
    _need(xs, "xs", torch.float32, 2)
    _need(w, "w", torch.int8, 2)
    _need(ws, "ws", torch.float32, 2)
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] with K = %d (got %s)" % (K, tuple(w.shape)))
    NB, KB = scale_shape(N, K, *block)
    if tuple(xs.shape) != (M, KB) or tuple(ws.shape) != (NB, KB):
        raise ValueError("scale shapes must be xs [M, %d] and ws [%d, %d]" % (KB, NB, KB))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must be [N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    nbytes = 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on a HIP device")
        nbytes = workspace.numel() * workspace.element_size()
    _check(load().blockint8_gemm_ws(_ptr(xq), _ptr(xs), _ptr(w), _ptr(ws), _ptr(bias), _ptr(y), M, N, K,
                                    block[0], block[1], _ptr(workspace), nbytes, _stream_handle(xq.device)))
    return y


def moe_gemm(xq: torch.Tensor, xs: torch.Tensor, expert_offsets: torch.Tensor, w: torch.Tensor,
             ws: torch.Tensor, y: torch.Tensor | None = None, block=(BLOCK, BLOCK),
             variant: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped block-scaled int8 GEMM over expert-sorted rows -> bf16 [R, N].

    ``expert_offsets`` is int32 [E+1] on the device (rows [off[e], off[e+1])
    use expert e); ``w`` is int8 [E, N, K], ``ws`` fp32 [E, ceil(N/128), ceil(K/128)].
    ``variant`` runs a named kernel (``GEMM_TILE_256X128`` or ``GEMM_TILE_256X256``).
    ``workspace`` (a contiguous device tensor of at least
    ``moe_gemm_workspace_size`` bytes; not with ``variant``) lets the tiles of
    a partial last round run split over K (``blockint8_moe_gemm_ws``).
    """
    _need(xq, "xq", torch.int8, 2)
    _need(xs, "xs", torch.float32, 2)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    _need(w, "w", torch.int8, 3)
    _need(ws, "ws", torch.float32, 3)
    R, K = xq.shape
    E, N, Kw = w.shape
    if Kw != K:
        raise ValueError("w must be [E, N, K] with K = %d" % K)
    if expert_offsets.shape[0] != E + 1:
        raise ValueError("expert_offsets must have E + 1 = %d entries" % (E + 1))
    NB, KB = scale_shape(N, K, *block)
    if tuple(xs.shape) != (R, KB) or tuple(ws.shape) != (E, NB, KB):
        raise ValueError("scale shapes must be xs [R, %d] and ws [E, %d, %d]" % (KB, NB, KB))
    if y is None:
        y = torch.empty((R, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (R, N):
        raise ValueError("y must be [R, N]")
    args = (_ptr(xq), _ptr(xs), _ptr(expert_offsets), _ptr(w), _ptr(ws), _ptr(y), R, N, K, E,
            block[0], block[1])
    if workspace is not None:
        if variant is not None:
            raise ValueError("a workspace runs the default kernel choice (no variant)")
        if (not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda"
                or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous tensor on a HIP device")
        nbytes = workspace.numel() * workspace.element_size()
        _check(load().blockint8_moe_gemm_ws(*args, _ptr(workspace), nbytes, _stream_handle(xq.device)))
    elif variant is None:
        _check(load().blockint8_moe_gemm(*args, _stream_handle(xq.device)))
    else:
        _check(load().blockint8_moe_gemm_variant(int(variant), *args, _stream_handle(xq.device)))
    return y


def moe_gemm_workspace_size(R: int, N: int, K: int, E: int, block=(BLOCK, BLOCK)) -> int:
    """Bytes of workspace ``moe_gemm`` can use for the grouped problem (0: none)."""
    return int(load().blockint8_moe_gemm_workspace_size(R, N, K, E, block[0], block[1]))


def linear(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor, bias: torch.Tensor | None = None,
           y: torch.Tensor | None = None, block=(BLOCK, BLOCK), xq: torch.Tensor | None = None,
           xs: torch.Tensor | None = None) -> torch.Tensor:
    """Block-wise INT8 linear with dynamic activation scales -> bf16 [M, N]:
    quant_act into the workspaces xq [M, K] int8 / xs [M, KB] fp32 (fresh
    tensors when not given; they hold the quantised activations on return),
    then gemm, through one C call."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.dtype != torch.bfloat16:
        raise TypeError("x must be a 2-D bfloat16 tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device; there is no CPU path")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    _need(w, "w", torch.int8, 2)
    _need(ws, "ws", torch.float32, 2)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] with K = %d (got %s)" % (K, tuple(w.shape)))
    NB, KB = scale_shape(N, K, *block)
    if tuple(ws.shape) != (NB, KB):
        raise ValueError("ws must be [%d, %d]" % (NB, KB))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must be [N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    _need(xq, "xq", torch.int8, 2)
    if tuple(xq.shape) != (M, K):
        raise ValueError("xq must be [%d, %d]" % (M, K))
    if xs is None:
        xs = torch.empty((M, KB), dtype=torch.float32, device=x.device)
    _need(xs, "xs", torch.float32, 2)
    if tuple(xs.shape) != (M, KB):
        raise ValueError("xs must be [%d, %d]" % (M, KB))
    ldx = x.stride(0) if M > 1 else K
    _check(load().blockint8_linear(_ptr(x), ldx, _ptr(w), _ptr(ws), _ptr(bias), _ptr(y), M, N, K,
                                   block[0], block[1], _ptr(xq), _ptr(xs), _stream_handle(x.device)))
    return y


def linear_noalloc(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor, bias: torch.Tensor | None = None,
                   y: torch.Tensor | None = None, block=(BLOCK, BLOCK)) -> torch.Tensor:
    """``linear`` with the quantised activations staged in the library's fixed
    per-GPU workspace (``NOALLOC_SCRATCH_BYTES``) instead of caller-given
    buffers: the C call allocates nothing.  Pass ``y`` to allocate nothing
    here either.  Calls that overlap in time on one GPU race (one stream is
    safe)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.dtype != torch.bfloat16:
        raise TypeError("x must be a 2-D bfloat16 tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device; there is no CPU path")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    _need(w, "w", torch.int8, 2)
    _need(ws, "ws", torch.float32, 2)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] with K = %d (got %s)" % (K, tuple(w.shape)))
    NB, KB = scale_shape(N, K, *block)
    if tuple(ws.shape) != (NB, KB):
        raise ValueError("ws must be [%d, %d]" % (NB, KB))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must be [N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    ldx = x.stride(0) if M > 1 else K
    _check(load().blockint8_linear_noalloc(_ptr(x), ldx, _ptr(w), _ptr(ws), _ptr(bias), _ptr(y), M, N, K,
                                           block[0], block[1], _stream_handle(x.device)))
    return y


# ----------------------------------------------------------------- MoE --

def moe_route(logits: torch.Tensor, k: int, renormalize: bool = False, out=None):
    """Top-k routing and dispatch order for fp32 router logits [T, E].

    Returns ``(topk_ids int32 [T, k], topk_weights fp32 [T, k], sorted_token
    int32 [T*k], expert_offsets int32 [E+1], row_of int32 [T, k])``, written
    into ``out`` (a tuple of those five tensors) when given."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T * k,), dtype=torch.int32, device=dev),
               torch.empty((E + 1,), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev))
    ids, w, st, off, row_of = out
    for t, name, dt, shape in ((ids, "topk_ids", torch.int32, (T, k)), (w, "topk_weights", torch.float32, (T, k)),
                               (st, "sorted_token", torch.int32, (T * k,)), (off, "expert_offsets", torch.int32, (E + 1,)),
                               (row_of, "row_of", torch.int32, (T, k))):
        _need(t, name, dt, len(shape))
        if tuple(t.shape) != shape:
            raise ValueError("%s must have shape %s" % (name, shape))
    _check(load().blockint8_moe_route(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(ids), _ptr(w),
                                      _ptr(st), _ptr(off), _ptr(row_of), _stream_handle(dev)))
    return ids, w, st, off, row_of


def quant_act_gather(x: torch.Tensor, rows: torch.Tensor, xq: torch.Tensor | None = None,
                     xs: torch.Tensor | None = None, block_k: int = BLOCK):
    """quant_act of the rows ``x[rows]`` (bf16 [T, K], int32 indices [R])."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.dtype != torch.bfloat16:
        raise TypeError("x must be a 2-D bfloat16 tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device; there is no CPU path")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    _need(rows, "rows", torch.int32, 1)
    T, K = x.shape
    R = rows.shape[0]
    KB = (K + block_k - 1) // block_k
    if xq is None:
        xq = torch.empty((R, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((R, KB), dtype=torch.float32, device=x.device)
    _need(xq, "xq", torch.int8, 2)
    _need(xs, "xs", torch.float32, 2)
    ldx = x.stride(0) if T > 1 else K
    _check(load().blockint8_quant_act_gather(_ptr(x), T, ldx, _ptr(rows), R, K, block_k, _ptr(xq), _ptr(xs),
                                             _stream_handle(x.device)))
    return xq, xs


def silu_mul_quant(h: torch.Tensor, aq: torch.Tensor | None = None, as_: torch.Tensor | None = None,
                   return_a: bool = False, block_k: int = BLOCK):
    """h = [gate | up] bf16 [R, 2I] -> (aq int8 [R, I], as fp32 [R, ceil(I/128)][, a bf16 [R, I]])."""
    _need(h, "h", torch.bfloat16, 2)
    R, two_i = h.shape
    if two_i % 2:
        raise ValueError("h must have an even number of columns (gate | up)")
    I = two_i // 2
    IB = (I + block_k - 1) // block_k
    if aq is None:
        aq = torch.empty((R, I), dtype=torch.int8, device=h.device)
    if as_ is None:
        as_ = torch.empty((R, IB), dtype=torch.float32, device=h.device)
    a = torch.empty((R, I), dtype=torch.bfloat16, device=h.device) if return_a else None
    _check(load().blockint8_silu_mul_quant(_ptr(h), R, I, block_k, _ptr(aq), _ptr(as_), _ptr(a),
                                           _stream_handle(h.device)))
    return (aq, as_, a) if return_a else (aq, as_)


def moe_gemm_silu_quant(xq: torch.Tensor, xs: torch.Tensor, expert_offsets: torch.Tensor, w13: torch.Tensor,
                        ws13: torch.Tensor, aq: torch.Tensor | None = None, as_: torch.Tensor | None = None,
                        block=(BLOCK, BLOCK)):
    """The w13 grouped GEMM with the SiLU gating and requantisation as its
    epilogue: (aq int8 [R, I], as fp32 [R, I/128]), bit-identical to
    silu_mul_quant(moe_gemm(xq, xs, expert_offsets, w13, ws13)).  w13 is
    int8 [E, 2I, K] (gate rows, then up rows); I % 128 == 0."""
    _need(xq, "xq", torch.int8, 2)
    _need(xs, "xs", torch.float32, 2)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    _need(w13, "w13", torch.int8, 3)
    _need(ws13, "ws13", torch.float32, 3)
    R, K = xq.shape
    E, N, Kw = w13.shape
    if Kw != K or N % 2:
        raise ValueError("w13 must be [E, 2I, K] with K = %d" % K)
    I = N // 2
    if expert_offsets.shape[0] != E + 1:
        raise ValueError("expert_offsets must have E + 1 = %d entries" % (E + 1))
    NB, KB = scale_shape(N, K, *block)
    if tuple(xs.shape) != (R, KB) or tuple(ws13.shape) != (E, NB, KB):
        raise ValueError("scale shapes must be xs [R, %d] and ws13 [E, %d, %d]" % (KB, NB, KB))
    IB = (I + block[1] - 1) // block[1]
    if aq is None:
        aq = torch.empty((R, I), dtype=torch.int8, device=xq.device)
    if as_ is None:
        as_ = torch.empty((R, IB), dtype=torch.float32, device=xq.device)
    _need(aq, "aq", torch.int8, 2)
    _need(as_, "as_", torch.float32, 2)
    if tuple(aq.shape) != (R, I) or tuple(as_.shape) != (R, IB):
        raise ValueError("aq must be [R, %d] and as_ [R, %d]" % (I, IB))
    _check(load().blockint8_moe_gemm_silu_quant(_ptr(xq), _ptr(xs), _ptr(expert_offsets), _ptr(w13), _ptr(ws13),
                                                _ptr(aq), _ptr(as_), R, I, K, E, block[0], block[1],
                                                _stream_handle(xq.device)))
    return aq, as_


def moe_combine(y2: torch.Tensor, row_of: torch.Tensor, topk_weights: torch.Tensor,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """out[t] = bf16(sum_s w[t, s] * y2[row_of[t, s]]) -> bf16 [T, H]."""
    _need(y2, "y2", torch.bfloat16, 2)
    _need(row_of, "row_of", torch.int32, 2)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    R, H = y2.shape
    T, k = row_of.shape
    if tuple(topk_weights.shape) != (T, k):
        raise ValueError("topk_weights must be [T, k] like row_of")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y2.device)
    _need(out, "out", torch.bfloat16, 2)
    _check(load().blockint8_moe_combine(_ptr(y2), R, _ptr(row_of), _ptr(topk_weights), T, k, H, _ptr(out),
                                        _stream_handle(y2.device)))
    return out


def moe_layer(x: torch.Tensor, logits: torch.Tensor, w13: torch.Tensor, ws13: torch.Tensor,
              w2: torch.Tensor, ws2: torch.Tensor, k: int, renormalize: bool = False,
              variant: int | None = None):
    """The block-wise INT8 FusedMoE layer on the GPU, one launch per step:
    route, gather + quantise, w13 grouped GEMM, SiLU gating + quantise, w2
    grouped GEMM, weighted combine.  With the default kernels and I % 128 == 0
    the w13 GEMM and the gating run as one launch (moe_gemm_silu_quant).  x bf16 [T, H]; logits fp32 [T, E];
    w13 int8 [E, 2I, H]; w2 int8 [E, H, I].  Returns bf16 [T, H]."""
    ids, w, st, off, row_of = moe_route(logits, k, renormalize)
    xq, xs = quant_act_gather(x, st)
    if variant is None and (w13.shape[1] // 2) % BLOCK == 0:
        aq, as_ = moe_gemm_silu_quant(xq, xs, off, w13, ws13)
    else:
        h = moe_gemm(xq, xs, off, w13, ws13, variant=variant)
        aq, as_ = silu_mul_quant(h)
    wsp = None
    if variant is None:
        nbytes = moe_gemm_workspace_size(aq.shape[0], w2.shape[1], aq.shape[1], w2.shape[0])
        wsp = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    y2 = moe_gemm(aq, as_, off, w2, ws2, variant=variant, workspace=wsp)
    return moe_combine(y2, row_of, w)


# ------------------------------------------------------- weight preparation --

def quant_weight(w: torch.Tensor, block=(BLOCK, BLOCK)):
    """Block quantisation of a bf16 weight [N, K] -> (int8 [N, K], fp32 [ceil(N/128), ceil(K/128)])."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2 or w.dtype != torch.bfloat16:
        raise TypeError("w must be a 2-D bfloat16 tensor")
    if w.device.type != "cuda":
        raise ValueError("w must be on a HIP device; there is no CPU path")
    if w.stride(1) != 1:
        raise ValueError("w rows must be contiguous (stride(1) == 1)")
    N, K = w.shape
    NB, KB = scale_shape(N, K, *block)
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    ws = torch.empty((NB, KB), dtype=torch.float32, device=w.device)
    ldw = w.stride(0) if N > 1 else K
    _check(load().blockint8_quant_weight(_ptr(w), N, K, ldw, block[0], block[1], _ptr(wq), _ptr(ws),
                                         _stream_handle(w.device)))
    return wq, ws


def check_tp_partition(input_size: int, input_size_per_partition: int, output_partition_sizes,
                       tp_size: int, block=(BLOCK, BLOCK)) -> None:
    """Raise BlockInt8Error unless the tensor-parallel partition boundaries
    fall on block boundaries (host only)."""
    sizes = (ctypes.c_int64 * len(output_partition_sizes))(*[int(v) for v in output_partition_sizes])
    _check(load().blockint8_check_tp_partition(int(input_size), int(input_size_per_partition), sizes,
                                               len(output_partition_sizes), int(tp_size), block[0], block[1]))
