"""The allocation-free linear (blockint8_linear_noalloc) against the linear
with caller-provided workspaces (blockint8_linear), through the C ABI.

Both run the same two launches, so y must be bit-identical; it is also
checked against the oracle within the GEMM tolerance.  Two calls in a row,
the second on a smaller problem (the library's per-GPU workspace keeps the
first call's contents), then the largest problem the workspace takes, the
per-channel form and a problem one row too large.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import oracle
import workloads as wl
from gpu_util import assert_gemm_close, bf16_bits, bf16_to_dev, device, to_dev

pytestmark = pytest.mark.gpu


def case(seed, M, N, K, bias=True, block=(128, 128)):
    rng = wl.rng_for(seed)
    x = wl.activations(rng, M, K, 0.01)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, *oracle.scale_shape(N, K, *block))
    b = wl.activations(rng, 1, N)[0] if bias else None
    return x, w, ws, b


def both(x, w, ws, b, block=(128, 128)):
    """(y from blockint8_linear_noalloc, y from blockint8_linear), each one C call."""
    lib = bi8.load()
    M, K = x.shape
    N = w.shape[0]
    KB = oracle.scale_shape(N, K, *block)[1]
    dev = device()
    xd, wd, wsd = bf16_to_dev(x), to_dev(w), to_dev(ws)
    bd = None if b is None else bf16_to_dev(b)
    y0 = torch.full((M, N), -1.0, dtype=torch.bfloat16, device=dev)
    y1 = torch.full((M, N), -2.0, dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty((M, KB), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = lib.blockint8_linear_noalloc(p(xd), K, p(wd), p(wsd), p(bd), p(y0), M, N, K, block[0], block[1], stream)
    assert st == 0, lib.blockint8_last_error().decode()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    st = lib.blockint8_linear(p(xd), K, p(wd), p(wsd), p(bd), p(y1), M, N, K, block[0], block[1], p(xq), p(xs),
                              stream)
    assert st == 0, lib.blockint8_last_error().decode()
    torch.cuda.synchronize()
    return bf16_bits(y0), bf16_bits(y1)


def check(x, w, ws, b, what, block=(128, 128)):
    y0, y1 = both(x, w, ws, b, block)
    assert np.array_equal(y0, y1), what + ": differs from blockint8_linear"
    xq, xs = oracle.quant_act(x, block_k=block[1])
    assert_gemm_close(y0, oracle.gemm(xq, xs, w, ws, bias=b, block=block), what)


def test_noalloc_linear_two_calls_second_smaller():
    check(*case(1, 300, 640, 1040), "first call, 300 x 640 x 1040 (tiled)")
    check(*case(2, 5, 300, 4000, bias=False), "second call, 5 x 300 x 4000 (skinny)")


def test_noalloc_linear_largest_problem_and_per_channel():
    # K = 4096: 4964 rows fill 20 MiB but for 1.7 KB; only rows sampled in
    # the oracle check
    x, w, ws, b = case(3, 4964, 256, 4096)
    y0, y1 = both(x, w, ws, b)
    assert np.array_equal(y0, y1)
    rows = np.array([0, 1234, 4095, 4963])
    q, s = oracle.quant_act(x[rows])
    assert_gemm_close(y0[rows], oracle.gemm(q, s, w, ws, bias=b), "4964 x 256 x 4096")
    K = 1024
    blk = (1, K)
    check(*case(4, 33, 520, K, block=blk), "per-channel 33 x 520 x 1024", block=blk)


def test_noalloc_linear_too_large_is_rejected_before_any_launch():
    x, w, ws, _ = case(5, 8, 128, 4096)
    xd = torch.zeros((4965, 4096), dtype=torch.bfloat16, device=device())
    with pytest.raises(bi8.BlockInt8Error, match="BI8_ERR_SHAPE"):
        bi8.linear_noalloc(xd, to_dev(w), to_dev(ws))
    # the binding's form of the call works on a problem that fits
    y = bi8.linear_noalloc(bf16_to_dev(x), to_dev(w), to_dev(ws))
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(bf16_bits(y), oracle.gemm(xq, xs, w, ws), "binding, 8 x 128 x 4096")
