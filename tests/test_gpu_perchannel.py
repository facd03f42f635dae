"""Parity of the per-channel W8A8 form (blocks of 1 x K: one scale per weight
row and one per token) with the CPU oracle's degenerate-block path.

Pages cited: "양자화 (Quantization)" (SGLang quantization page: the w8a8_int8
and auto-round-int8 schemes, per-channel weights with per-token dynamic
activations) and "[SGLang] Block-wise INT8: 블록 단위 정수 양자화", section 2 (the
scale tensor [ceil(N/bn), ceil(K/bk)], here [N, 1]).
"""
import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import oracle
import workloads as wl
from gpu_util import assert_gemm_close, bf16_bits, bf16_to_dev, device, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 16), (8, 4096), (300, 4000), (5, 131072), (64, 2064)])
def test_per_token_quant_bit_exact(M, K):
    x = wl.activations(np.random.default_rng(M + K), M, K, 0.01)
    xq, xs = bi8.quant_act(bf16_to_dev(x), block_k=K)
    q_ref, s_ref = oracle.quant_act(x, block_k=K)
    assert xs.shape == (M, 1)
    assert np.array_equal(xq.cpu().numpy(), q_ref) and np.array_equal(xs.cpu().numpy(), s_ref)


def pc_case(seed, M, N, K):
    rng = wl.rng_for(seed)
    x = wl.activations(rng, M, K)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, N, 1)
    return x, w, ws


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (8, 4096, 4096), (200, 1000, 1040), (513, 520, 4000),
                                   (4096, 4096, 4096), (33, 7, 16), (4000, 4100, 1040),
                                   (40, 1000, 1040), (64, 520, 2064), (24, 28672, 256)])
def test_per_channel_gemm_vs_oracle(M, N, K):
    x, w, ws = pc_case((M, N, K, 1), M, N, K)
    xq, xs = oracle.quant_act(x, block_k=K)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws), block=(1, K)))
    rows = np.arange(M) if M * N * K < 2 ** 31 else np.linspace(0, M - 1, 24).astype(int)
    y_ref = oracle.gemm(xq[rows], xs[rows], w, ws, block=(1, K))
    assert_gemm_close(y[rows], y_ref, "per-channel M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(40, 300, 1040), (130, 64, 528), (1300, 11002, 272)])
def test_per_channel_integer_closed_form_bit_exact(M, N, K):
    """Unit scales: y is the integer product rounded once to bf16.  The sums
    stay below 127^2 * K < 2^53, so the float64 product is exact.  The last
    shape has 6 x 43 tiles of 256 x 256, an odd count of 128-wide K blocks
    with a ragged tail, and an N that rules out 4-wide stores."""
    rng = np.random.default_rng(M * N)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    exact = (xq.astype(np.float64) @ w.astype(np.float64).T).astype(np.float32)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(np.ones((M, 1), np.float32)), to_dev(w),
                           to_dev(np.ones((N, 1), np.float32)), block=(1, K)))
    assert np.array_equal(y, wl.to_bf16_bits(exact))


def test_per_channel_linear_and_bias():
    M, N, K = 70, 333, 2048
    x, w, ws = pc_case(5, M, N, K)
    bias = wl.activations(np.random.default_rng(2), 1, N)[0]
    y = bf16_bits(bi8.linear(bf16_to_dev(x), to_dev(w), to_dev(ws), bias=bf16_to_dev(bias), block=(1, K)))
    xq, xs = oracle.quant_act(x, block_k=K)
    assert_gemm_close(y, oracle.gemm(xq, xs, w, ws, bias=bias, block=(1, K)), "per-channel linear")


@pytest.mark.parametrize("M", [8, 40])
def test_per_channel_max_k_saturated_sums_bit_exact(M):
    """K = 2^17, the per-channel limit, with every code at +-127: a row's int32
    sum reaches +-127^2 * 2^17 = +-2114060288, just inside int32 (M = 8 runs
    the skinny kernel, M = 40 the tiled one).  All partial sums are exact in
    fp32 here, so y must equal the oracle bit for bit."""
    N, K = 64, 1 << 17
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    w = np.full((N, K), 127, np.int8)
    w[::3] = -127
    xs = np.ones((M, 1), np.float32)
    ws = np.ones((N, 1), np.float32)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws), block=(1, K)))
    y_ref = oracle.gemm(xq, xs, w, ws, block=(1, K))
    assert abs(int(xq[0].astype(np.int64) @ w[1].astype(np.int64))) == 127 * 127 * K
    assert np.array_equal(y, y_ref)


def test_per_channel_max_k_saturated_sums_many_tiles():
    """K = 2^17 with every code at +-127 on 16 x 16 tiles of 256 x 256: each
    output is +-127^2 * 2^17 exactly, with the sign of its token row times
    the sign of its weight row."""
    M = N = 4096
    K = 1 << 17
    sm = np.where(np.arange(M) % 2 == 1, -1, 1).astype(np.int8)
    sn = np.where(np.arange(N) % 3 == 0, -1, 1).astype(np.int8)
    xq = np.repeat((127 * sm)[:, None], K, axis=1)
    w = np.repeat((127 * sn)[:, None], K, axis=1)
    y = bf16_bits(bi8.gemm(to_dev(xq), to_dev(np.ones((M, 1), np.float32)), to_dev(w),
                           to_dev(np.ones((N, 1), np.float32)), block=(1, K)))
    del xq, w
    exact = np.outer(sm.astype(np.float32), sn.astype(np.float32)) * np.float32(127 * 127 * K)
    assert np.array_equal(y, wl.to_bf16_bits(exact))
