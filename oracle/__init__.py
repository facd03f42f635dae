"""CPU oracle for the block-wise INT8 W8A8 linear layer -- test infrastructure.

This package is the reference the GPU path is checked against.  It is NOT part
of the product: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
``block_wise_int8_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain scalar C, built with gcc, no
fast-math, no FMA contraction); this module only marshals numpy arrays.
Pages cited: "[SGLang] Block-wise INT8: 블록 단위 정수 양자화"
(blog.secrett2633.cloud), sections as named in each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (with ``sanitize``,
    under AddressSanitizer and UndefinedBehaviorSanitizer, for the host
    sanitizer run of the CPU tests)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g"] if sanitize else []
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fno-finite-math-only", "-shared", "-fPIC"] + san + ["-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_scale_shape.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.oracle_quant_act.argtypes = [vp, i64, i64, i64, i64, vp, vp]
    lib.oracle_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64]
    lib.oracle_gemm_f64.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64]
    lib.oracle_moe_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64]
    lib.oracle_quant_weight.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp]
    lib.oracle_topk_softmax.argtypes = [vp, i64, i64, i64, ctypes.c_int, vp, vp]
    lib.oracle_moe_align.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.oracle_silu_mul.argtypes = [vp, i64, i64, vp]
    lib.oracle_combine.argtypes = [vp, i64, vp, vp, i64, i64, i64, vp]
    for f in ("oracle_scale_shape", "oracle_quant_act", "oracle_gemm", "oracle_gemm_f64",
              "oracle_moe_gemm", "oracle_quant_weight", "oracle_topk_softmax", "oracle_moe_align", "oracle_silu_mul",
              "oracle_combine"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed (code %d)" % (what, rc))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f64_to_bf16(v: float) -> int:
    """One RNE rounding of a binary64 value to bf16 bits."""
    return int(_load().oracle_f64_to_bf16(float(v)))


def bf16_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(b) & 0xFFFF))


def scale_shape(N: int, K: int, block_n: int = 128, block_k: int = 128):
    """[BW8] §2: shape of the fp32 block-scale tensor of an int8 [N, K] weight."""
    r, c = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().oracle_scale_shape(N, K, block_n, block_k, ctypes.byref(r), ctypes.byref(c)),
           "scale_shape")
    return int(r.value), int(c.value)


def quant_act(x_bf16: np.ndarray, block_k: int = 128, K: int | None = None):
    """[BW8] §4: dynamic per-(token, K-group) activation quantisation.

    ``x_bf16``: uint16 bf16 bits [M, ldx]; ``K`` (default ldx) columns are used.
    Returns (xq int8 [M, K], xs float32 [M, ceil(K/block_k)]).
    """
    x = _c(x_bf16, np.uint16)
    M, ldx = x.shape
    K = ldx if K is None else K
    KB = (K + block_k - 1) // block_k if K > 0 else 0
    xq = np.zeros((M, K), np.int8)
    xs = np.zeros((M, KB), np.float32)
    _check(_load().oracle_quant_act(_ptr(x), M, K, ldx, block_k, _ptr(xq), _ptr(xs)), "quant_act")
    return xq, xs


def _gemm_args(xq, xs, w, ws, bias):
    xq, xs, w, ws = _c(xq, np.int8), _c(xs, np.float32), _c(w, np.int8), _c(ws, np.float32)
    bias = None if bias is None else _c(bias, np.uint16)
    return xq, xs, w, ws, bias


def gemm(xq, xs, w, ws, bias=None, block=(128, 128)) -> np.ndarray:
    """[BW8] §2/§4: y = bf16( sum_g int_dot_g * xs * ws (+ bias) ), bf16 bits [M, N]."""
    xq, xs, w, ws, bias = _gemm_args(xq, xs, w, ws, bias)
    M, K = xq.shape
    N = w.shape[0]
    y = np.zeros((M, N), np.uint16)
    _check(_load().oracle_gemm(_ptr(xq), _ptr(xs), _ptr(w), _ptr(ws), _ptr(bias), _ptr(y),
                               M, N, K, block[0], block[1]), "gemm")
    return y


def gemm_f64(xq, xs, w, ws, bias=None, block=(128, 128)) -> np.ndarray:
    """The same sum as :func:`gemm`, before the bf16 rounding (float64 [M, N])."""
    xq, xs, w, ws, bias = _gemm_args(xq, xs, w, ws, bias)
    M, K = xq.shape
    N = w.shape[0]
    y = np.zeros((M, N), np.float64)
    _check(_load().oracle_gemm_f64(_ptr(xq), _ptr(xs), _ptr(w), _ptr(ws), _ptr(bias), _ptr(y),
                                   M, N, K, block[0], block[1]), "gemm_f64")
    return y


def moe_gemm(xq, xs, offsets, w, ws, block=(128, 128)) -> np.ndarray:
    """[BW8] §5/§6: per-expert O2 over rows sorted by expert.

    ``offsets``: int32 [E+1]; ``w``: int8 [E, N, K]; ``ws``: fp32 [E, NB, KB].
    """
    xq, xs, w, ws, _ = _gemm_args(xq, xs, w, ws, None)
    off = _c(offsets, np.int32)
    R, K = xq.shape
    E, N, _ = w.shape
    y = np.zeros((R, N), np.uint16)
    _check(_load().oracle_moe_gemm(_ptr(xq), _ptr(xs), _ptr(off), _ptr(w), _ptr(ws), _ptr(y),
                                   R, N, K, E, block[0], block[1]), "moe_gemm")
    return y


def quant_weight(w_bf16, block=(128, 128), K: int | None = None):
    """Block quantisation of a bf16 weight [N, ldw] (``K`` columns, default ldw).

    Returns (wq int8 [N, K], ws float32 [ceil(N/bn), ceil(K/bk)])."""
    w = _c(w_bf16, np.uint16)
    N, ldw = w.shape
    K = ldw if K is None else K
    NB = (N + block[0] - 1) // block[0] if N > 0 else 0
    KB = (K + block[1] - 1) // block[1] if K > 0 else 0
    wq = np.zeros((N, K), np.int8)
    ws = np.zeros((NB, KB), np.float32)
    _check(_load().oracle_quant_weight(_ptr(w), N, K, ldw, block[0], block[1], _ptr(wq), _ptr(ws)),
           "quant_weight")
    return wq, ws


# ------------------------------------------------------------ MoE steps --

def topk_softmax(logits, k: int, renorm: bool = False):
    """Router: top-k of the binary64 softmax of fp32 logits [T, E].

    Returns (ids int32 [T, k] in pick order, weights float64 [T, k]); ties
    go to the lower expert; ``renorm`` divides the k weights by their sum."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    _check(_load().oracle_topk_softmax(_ptr(lg), T, E, k, int(bool(renorm)), _ptr(ids), _ptr(w)),
           "topk_softmax")
    return ids, w


def moe_align(ids, E: int):
    """Dispatch order of the rows (t, slot), stable by (expert, t, slot).

    Returns (sorted_token int32 [T*k], offsets int32 [E+1], row_of int32 [T, k])."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    st = np.zeros(T * k, np.int32)
    off = np.zeros(E + 1, np.int32)
    row_of = np.zeros((T, k), np.int32)
    _check(_load().oracle_moe_align(_ptr(ids), T, k, E, _ptr(st), _ptr(off), _ptr(row_of)), "moe_align")
    return st, off, row_of


def silu_mul(h_bf16):
    """a = bf16(silu(gate) * up) for h = [gate | up], bf16 bits [R, 2I] -> [R, I]."""
    h = _c(h_bf16, np.uint16)
    R, two_i = h.shape
    I = two_i // 2
    a = np.zeros((R, I), np.uint16)
    _check(_load().oracle_silu_mul(_ptr(h), R, I, _ptr(a)), "silu_mul")
    return a


def combine(y2_bf16, row_of, weights):
    """out[t] = bf16(sum_s w[t, s] * y2[row_of[t, s]]), bf16 bits [T, H]."""
    y2 = _c(y2_bf16, np.uint16)
    ro = _c(row_of, np.int32)
    w = _c(weights, np.float32)
    T, k = ro.shape
    R, H = y2.shape
    out = np.zeros((T, H), np.uint16)
    _check(_load().oracle_combine(_ptr(y2), R, _ptr(ro), _ptr(w), T, k, H, _ptr(out)), "combine")
    return out
