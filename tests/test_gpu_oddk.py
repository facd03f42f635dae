"""K not a multiple of 16 (and rows at any alignment) through the C ABI.

Section 2 of the page "[SGLang] Block-wise INT8" (blog.secrett2633.cloud)
sizes the block-scale tensor with a ceiling for any input size, so the last
K group may hold any number of entries from 1 to 128.  With K % 16 != 0 the
int8 rows of xq and w start at any byte: the quantisers read and write such
rows element by element where a 16-byte move would be unaligned, and the GEMM
runs one alignment-safe kernel (every shape; tokens in chunks of 64).  Codes
and scales must match the oracle bit-exactly, GEMM outputs within the GEMM
tolerance, and integer cases bit-exactly.
"""
import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import oracle
import workloads as wl
from gpu_util import assert_gemm_close, bf16_bits, bf16_to_dev, device, to_dev

pytestmark = pytest.mark.gpu

ODD_K = [1, 7, 17, 24, 130, 1000, 4001, 4095]


def strided_dev(x, pad, offset=0):
    """x [M, K] on the device inside a wider buffer: row stride K + pad,
    starting `offset` elements into the buffer (an unaligned base)."""
    M, K = x.shape
    buf = torch.zeros((M * (K + pad) + offset + 8,), dtype=torch.bfloat16, device=device())
    v = buf[offset:offset + M * (K + pad)].view(M, K + pad)[:, :K]
    v.copy_(bf16_to_dev(x))
    return v


@pytest.mark.parametrize("K", ODD_K)
@pytest.mark.parametrize("M", [1, 5, 70])
def test_quant_any_k_bit_exact(M, K):
    x = wl.activations(np.random.default_rng(M * 31 + K), M, K, 0.02)
    q_ref, s_ref = oracle.quant_act(x)
    for pad, off in ((0, 0), (3, 0), (5, 1)):   # dense, odd stride, odd stride and base
        xd = strided_dev(x, pad, off)
        xq, xs = bi8.quant_act(xd)
        assert np.array_equal(xq.cpu().numpy(), q_ref), (pad, off)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), (pad, off)


@pytest.mark.parametrize("K", [17, 1000, 4001, 4095, 9001])
def test_quant_per_token_any_k_bit_exact(K):
    M = 9
    x = wl.activations(np.random.default_rng(K), M, K, 0.02)
    q_ref, s_ref = oracle.quant_act(x, block_k=K)
    for pad, off in ((0, 0), (3, 1)):
        xq, xs = bi8.quant_act(strided_dev(x, pad, off), block_k=K)
        assert np.array_equal(xq.cpu().numpy(), q_ref) and np.array_equal(xs.cpu().numpy(), s_ref)


@pytest.mark.parametrize("K", [17, 4001])
def test_quant_gather_any_k_bit_exact(K):
    T = 50
    rng = np.random.default_rng(K + 5)
    x = wl.activations(rng, T, K)
    rows = rng.integers(0, T, 120).astype(np.int32)
    xq, xs = bi8.quant_act_gather(strided_dev(x, 3), to_dev(rows))
    q_ref, s_ref = oracle.quant_act(x[rows])
    assert np.array_equal(xq.cpu().numpy(), q_ref) and np.array_equal(xs.cpu().numpy(), s_ref)


# every token-tile count of the kernel (M <= 16, 32, 48, 64) and several
# 64-token chunks, ragged N, K groups from 1 to 127 entries long
GEMM_ODD = [(1, 16, 17), (8, 300, 4001), (16, 256, 4095), (20, 130, 1), (33, 200, 130), (48, 64, 7),
            (64, 520, 4095), (65, 333, 17), (200, 1000, 4001), (333, 520, 1000)]


@pytest.mark.parametrize("M,N,K", GEMM_ODD)
def test_gemm_any_k_vs_oracle(M, N, K):
    rng = wl.rng_for((M, N, K, 9))
    x = wl.activations(rng, M, K, 0.01)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, *oracle.scale_shape(N, K))
    xq, xs = oracle.quant_act(x)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws)))
    assert_gemm_close(y, oracle.gemm(xq, xs, w, ws), "M=%d N=%d K=%d" % (M, N, K))
    if K % 16:
        for v in (bi8.GEMM_SKINNY, bi8.GEMM_TILE_128X64, bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256):
            with pytest.raises(bi8.BlockInt8Error, match="BI8_ERR_ALIGN"):
                bi8.gemm(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws), variant=v)


@pytest.mark.parametrize("M,N,K", [(5, 300, 1039), (70, 260, 1001), (130, 64, 17)])
def test_gemm_any_k_integer_closed_form_bit_exact(M, N, K):
    """Unit scales and integer activations at odd K: y == bf16(int64 matmul)."""
    rng = np.random.default_rng(M + N + K)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    NB, KB = oracle.scale_shape(N, K)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(np.ones((M, KB), np.float32)), to_dev(w),
                           to_dev(np.ones((NB, KB), np.float32))))
    exact = (xq.astype(np.int64) @ w.astype(np.int64).T).astype(np.float32)
    assert np.array_equal(y, wl.to_bf16_bits(exact))


@pytest.mark.parametrize("M,N,K", [(8, 300, 4001), (100, 520, 1001)])
def test_gemm_per_channel_any_k(M, N, K):
    rng = wl.rng_for((M, N, K, 11))
    x = wl.activations(rng, M, K)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, N, 1)
    xq, xs = oracle.quant_act(x, block_k=K)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws), block=(1, K)))
    assert_gemm_close(y, oracle.gemm(xq, xs, w, ws, block=(1, K)), "per-channel K=%d" % K)


@pytest.mark.parametrize("M,N,K", [(5, 300, 4001), (90, 256, 17)])
def test_linear_any_k_with_stride(M, N, K):
    """Both linears, x with an odd row stride and an odd base, with bias."""
    rng = wl.rng_for((M, N, K, 13))
    x = wl.activations(rng, M, K, 0.01)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, *oracle.scale_shape(N, K))
    b = wl.activations(rng, 1, N)[0]
    xd = strided_dev(x, 3, 1)
    wd, wsd, bd = to_dev(w), to_dev(ws), bf16_to_dev(b)
    y1 = bf16_bits(bi8.linear(xd, wd, wsd, bias=bd))
    y2 = bf16_bits(bi8.linear_noalloc(xd, wd, wsd, bias=bd))
    assert np.array_equal(y1, y2)
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(y1, oracle.gemm(xq, xs, w, ws, bias=b), "linear K=%d" % K)


def test_grouped_gemm_keeps_k_multiple_of_16():
    xq = torch.zeros((4, 17), dtype=torch.int8, device=device())
    xs = torch.ones((4, 1), dtype=torch.float32, device=device())
    w = torch.zeros((2, 16, 17), dtype=torch.int8, device=device())
    ws = torch.ones((2, 1, 1), dtype=torch.float32, device=device())
    off = torch.tensor([0, 2, 4], dtype=torch.int32, device=device())
    with pytest.raises(bi8.BlockInt8Error, match="BI8_ERR_ALIGN"):
        bi8.moe_gemm(xq, xs, off, w, ws)
