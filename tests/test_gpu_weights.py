"""Parity of the offline block weight quantiser with the CPU oracle (bit-exact
codes and scales), and the quantise-then-GEMM pipeline.

Page cited: "[SGLang] Block-wise INT8: 블록 단위 정수 양자화" (blog.secrett2633.cloud),
sections 1 and 2.
"""
import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import oracle
import workloads as wl
from gpu_util import assert_gemm_close, bf16_bits, bf16_to_dev, device, to_dev

pytestmark = pytest.mark.gpu


def gpu_qw(w_bits, ldw=None):
    N, K = w_bits.shape
    if ldw is None:
        wq, ws = bi8.quant_weight(bf16_to_dev(w_bits))
    else:
        wd = torch.zeros((N, ldw), dtype=torch.bfloat16, device=device())
        wd[:, :K] = bf16_to_dev(w_bits)
        wq, ws = bi8.quant_weight(wd[:, :K])
    return wq.cpu().numpy(), ws.cpu().numpy()


@pytest.mark.parametrize("N,K", [(128, 128), (300, 400), (4096, 4096), (5000, 4000), (1, 16), (129, 4112)])
def test_quant_weight_bit_exact(N, K):
    w = wl.activations(np.random.default_rng(N + K), N, K, 0.01)
    wq, ws = gpu_qw(w)
    wq_r, ws_r = oracle.quant_weight(w)
    assert np.array_equal(wq, wq_r) and np.array_equal(ws, ws_r)


def test_quant_weight_row_stride_and_special_blocks():
    rng = np.random.default_rng(5)
    w = wl.activations(rng, 256, 384)
    w[:128, :128] = 0                                                          # zero block
    w[128:, :128] = wl.to_bf16_bits(np.full((128, 128), 3e-39, np.float32))   # subnormal block
    blk = np.zeros((128, 128), np.float32)
    blk[0, :6] = [0.5, 1.5, 2.5, -2.5, 126.5, 127.0]                            # ties at s = 1
    w[:128, 128:256] = wl.to_bf16_bits(blk)
    wq, ws = gpu_qw(w, ldw=392)
    wq_r, ws_r = oracle.quant_weight(w)
    assert np.array_equal(wq, wq_r) and np.array_equal(ws, ws_r)
    assert ws[0, 1] == 1.0 and wq[0, 128:134].tolist() == [0, 2, 2, -2, 126, 127]


def test_quantised_weights_drive_the_gemm():
    """bf16 weight -> quant_weight -> gemm equals the oracle's quantiser and GEMM."""
    rng = np.random.default_rng(6)
    M, N, K = 200, 640, 1040
    wb = wl.activations(rng, N, K)
    x = wl.activations(rng, M, K)
    wq, ws = bi8.quant_weight(bf16_to_dev(wb))
    y = bf16_bits(bi8.linear(bf16_to_dev(x), wq, ws))
    wq_r, ws_r = oracle.quant_weight(wb)
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(y, oracle.gemm(xq, xs, wq_r, ws_r), "quantised weights")
