"""Helpers shared by the GPU tests: host<->device marshalling and comparisons.

Holds none of the method's arithmetic: expected values always come from the
oracle (or a library routine in a pin), never from here.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

# Tolerance for the GEMM outputs: max |y_gpu - y_ref| / max |y_ref| per output
# tensor.  The fp32 kernels and the fp64 oracle see identical int8 inputs and
# scales; only the order and precision of the fp32 accumulation differ.
GEMM_REL_TOL = 1e-2


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible HIP device")
    return torch.device("cuda:0")


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ordered(b: np.ndarray) -> np.ndarray:
    """Map bf16 bits to integers whose differences count ulps."""
    b = np.asarray(b, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def gemm_report(y_gpu: np.ndarray, y_ref: np.ndarray):
    g, r = bits_to_f64(y_gpu), bits_to_f64(y_ref)
    scale = max(np.abs(r).max(initial=0.0), 1e-30)
    rel = np.abs(g - r).max(initial=0.0) / scale
    ulp = np.abs(ordered(y_gpu) - ordered(y_ref))
    return rel, float(np.mean(ulp > 1)) if ulp.size else 0.0, int(ulp.max(initial=0))


def assert_gemm_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(bits_to_f64(y_gpu))), what + ": non-finite output"
    rel, frac_gt1, maxulp = gemm_report(y_gpu, y_ref)
    assert rel <= GEMM_REL_TOL, "%s: max rel err %.3e > %.0e" % (what, rel, GEMM_REL_TOL)
    # Sanity beyond the tolerance: identical int8 inputs leave only fp32
    # rounding, so almost every element is within 1 bf16 ulp.
    assert frac_gt1 <= 0.01, "%s: %.3f%% of outputs more than 1 ulp apart" % (what, 100 * frac_gt1)
    return rel, frac_gt1, maxulp


def host_threads() -> int:
    """CPU threads this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_gemm_rows(xq, xs, w, ws, bias=None):
    """oracle.gemm on the given activation rows, split into row slices run on
    a thread pool (the oracle call itself is unchanged and single-threaded;
    each slice is an independent call on disjoint rows)."""
    oracle.scale_shape(1, 1)   # load the library once, before the threads
    M = xq.shape[0]
    n = min(host_threads(), max(1, M))
    bounds = np.linspace(0, M, n + 1).astype(int)
    parts = [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    with ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(lambda ab: oracle.gemm(xq[ab[0]:ab[1]], xs[ab[0]:ab[1]], w, ws, bias=bias), parts))
    return np.concatenate(outs) if outs else np.zeros((0, w.shape[0]), np.uint16)
