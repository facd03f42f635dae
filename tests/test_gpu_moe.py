"""Parity of the MoE steps around the grouped GEMM with the CPU oracle.

Routing decisions, dispatch order and quantised codes must match exactly.
Stage-wise: each GPU stage is checked against the oracle fed the GPU's own
previous-stage output, so that a last-ulp difference in the fp32 SiLU or
combine (the oracle works in binary64) cannot masquerade as a quantisation
error.  Those two bf16 results must agree to within one bf16 ulp everywhere
and exactly almost everywhere.

Page cited: "[SGLang] Block-wise INT8: 블록 단위 정수 양자화" (blog.secrett2633.cloud),
sections 5 and 6.
"""
import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import oracle
import workloads as wl
from gpu_util import (GEMM_REL_TOL, bf16_bits, bf16_to_dev, bits_to_f64, device, gemm_report, ordered,
                      to_dev)

pytestmark = pytest.mark.gpu


def route_both(logits, k, renorm=False):
    ids, w, st, off, row_of = bi8.moe_route(to_dev(logits), k, renorm)
    gpu = [t.cpu().numpy() for t in (ids, w, st, off, row_of)]
    ids_r, w_r = oracle.topk_softmax(logits, k, renorm)
    st_r, off_r, row_of_r = oracle.moe_align(ids_r, logits.shape[1])
    return gpu, (ids_r, w_r, st_r, off_r, row_of_r)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (7, 3, 1), (1000, 8, 2), (4096, 8, 2), (2500, 64, 4),
                                   (333, 16, 8), (5, 1, 1), (1025, 128, 2), (3000, 65, 2), (4096, 512, 8)])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_matches_oracle(T, E, k, renorm):
    logits = wl.router_logits(np.random.default_rng(T * 31 + E), T, E)
    (ids, w, st, off, row_of), (ids_r, w_r, st_r, off_r, row_of_r) = route_both(logits, k, renorm)
    assert np.array_equal(ids, ids_r)
    np.testing.assert_allclose(w, w_r, rtol=2e-6, atol=1e-30)
    assert np.array_equal(off, off_r)
    assert np.array_equal(st, st_r)
    assert np.array_equal(row_of, row_of_r)


def test_route_ties_go_to_the_lower_expert():
    rng = np.random.default_rng(3)
    logits = (np.round(rng.standard_normal((512, 8)) * 2) / 2).astype(np.float32)   # many exact ties
    logits[0] = 0.0
    (ids, _, st, off, row_of), (ids_r, _, st_r, off_r, row_of_r) = route_both(logits, 2)
    assert np.array_equal(ids, ids_r) and ids[0].tolist() == [0, 1]
    assert np.array_equal(st, st_r) and np.array_equal(off, off_r) and np.array_equal(row_of, row_of_r)


def test_route_empty_batch():
    off = bi8.moe_route(torch.zeros((0, 8), dtype=torch.float32, device=device()), 2)[3]
    assert off.cpu().numpy().tolist() == [0] * 9


@pytest.mark.parametrize("T,K", [(64, 256), (300, 4000), (17, 16)])
def test_quant_act_gather_is_gather_of_quant(T, K):
    rng = np.random.default_rng(T + K)
    x = wl.activations(rng, T, K, 0.01)
    rows = rng.integers(0, T, 3 * T).astype(np.int32)
    xq, xs = bi8.quant_act_gather(bf16_to_dev(x), to_dev(rows))
    q_ref, s_ref = oracle.quant_act(x[rows])
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy(), s_ref)


def test_quant_act_gather_out_of_range_rows_read_zero():
    x = wl.activations(np.random.default_rng(1), 8, 128)
    rows = np.array([0, -1, 8, 7], np.int32)
    xq, xs = bi8.quant_act_gather(bf16_to_dev(x), to_dev(rows))
    xq, xs = xq.cpu().numpy(), xs.cpu().numpy()
    assert np.all(xq[1:3] == 0) and np.all(xs[1:3] == 0)
    q_ref, s_ref = oracle.quant_act(x[[0, 7]])
    assert np.array_equal(xq[[0, 3]], q_ref) and np.array_equal(xs[[0, 3]], s_ref)


def assert_bf16_near(got, ref, what, exact_frac=0.999):
    d = np.abs(ordered(got) - ordered(ref))
    assert d.max(initial=0) <= 1, "%s: %d ulp apart" % (what, d.max())
    assert np.mean(d == 0) >= exact_frac, "%s: only %.5f exact" % (what, np.mean(d == 0))


@pytest.mark.parametrize("R,I", [(8, 128), (100, 14336), (33, 400), (1, 16)])
def test_silu_mul_quant_stagewise(R, I):
    rng = np.random.default_rng(R * I)
    h = wl.activations(rng, R, 2 * I)
    h_big = wl.to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32) * 40)
    for hh in (h, h_big):
        aq, as_, a = bi8.silu_mul_quant(bf16_to_dev(hh), return_a=True)
        a = bf16_bits(a)
        assert_bf16_near(a, oracle.silu_mul(hh), "silu*up", exact_frac=0.995)
        q_ref, s_ref = oracle.quant_act(a)                       # stage-wise: the GPU's own a
        assert np.array_equal(aq.cpu().numpy(), q_ref)
        assert np.array_equal(as_.cpu().numpy(), s_ref)
        aq2, as2 = bi8.silu_mul_quant(bf16_to_dev(hh))             # without the optional copy
        assert torch.equal(aq2, aq) and torch.equal(as2, as_)


def test_silu_mul_quant_special_values():
    g = np.array([0.0, -0.0, 1.0, -1.0, 88.0, -88.0, 200.0, -200.0, 1e-30, -3e4] + [0.5] * 6, np.float32)
    u = np.array([1.0, 2.0, 0.0, -3.0, 1.0, 1.0, -1.0, 5.0, 1.0, 1.0] + [2.0] * 6, np.float32)
    h = np.concatenate([wl.to_bf16_bits(g), wl.to_bf16_bits(u)])[None, :]
    aq, as_, a = bi8.silu_mul_quant(bf16_to_dev(h), return_a=True)
    assert_bf16_near(bf16_bits(a), oracle.silu_mul(h), "special", exact_frac=0.9)
    q_ref, s_ref = oracle.quant_act(bf16_bits(a))
    assert np.array_equal(aq.cpu().numpy(), q_ref) and np.array_equal(as_.cpu().numpy(), s_ref)


@pytest.mark.parametrize("T,E,k,H", [(64, 8, 2, 256), (1000, 16, 4, 4096), (3, 2, 1, 8)])
def test_combine_stagewise(T, E, k, H):
    rng = np.random.default_rng(T + H)
    logits = wl.router_logits(rng, T, E)
    _, w, _, _, row_of = bi8.moe_route(to_dev(logits), k)
    y2 = wl.activations(rng, T * k, H)
    out = bf16_bits(bi8.moe_combine(bf16_to_dev(y2), row_of, w))
    ro, wn = row_of.cpu().numpy(), w.cpu().numpy()
    ref = oracle.combine(y2, ro, wn)   # the GPU's routing
    # fp32 against binary64: beyond the bf16 rounding, the fp32 sum of k terms
    # may be off by k rounding errors of the terms' magnitude (cancellation)
    g, r = bits_to_f64(out), bits_to_f64(ref)
    mag = np.abs(wn[:, :, None].astype(np.float64) * bits_to_f64(y2)[ro]).sum(axis=1)
    ulp = np.abs(r) * 2.0 ** -7 + 2.0 ** -133   # one bf16 ulp or more
    assert np.all(np.abs(g - r) <= ulp + k * 2.0 ** -23 * mag), "combine outside the fp32 bound"
    assert np.mean(out == ref) >= 0.99


def oracle_moe_layer(x, logits, w13, ws13, w2, ws2, k):
    T, H = x.shape
    E = logits.shape[1]
    ids, wts = oracle.topk_softmax(logits, k)
    st, off, row_of = oracle.moe_align(ids, E)
    xq, xs = oracle.quant_act(x[st])
    h = oracle.moe_gemm(xq, xs, off, w13, ws13)
    a = oracle.silu_mul(h)
    aq, as_ = oracle.quant_act(a)
    y2 = oracle.moe_gemm(aq, as_, off, w2, ws2)
    return oracle.combine(y2, row_of, wts.astype(np.float32))


@pytest.mark.parametrize("T,H,I,E,k", [(96, 256, 384, 4, 2), (200, 512, 256, 8, 2), (40, 128, 128, 3, 1)])
@pytest.mark.parametrize("variant", [None, bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256])
def test_moe_layer_end_to_end(T, H, I, E, k, variant):
    """The whole FusedMoE layer against the oracle's pipeline (GEMM tolerance:
    the fp32 SiLU may move a requantised code by one)."""
    rng = np.random.default_rng(T + H + I)
    x = wl.activations(rng, T, H)
    logits = wl.router_logits(rng, T, E)
    w13 = wl.weights(rng, E, 2 * I, H)
    ws13 = wl.weight_scales(rng, E, *oracle.scale_shape(2 * I, H))
    w2 = wl.weights(rng, E, H, I)
    ws2 = wl.weight_scales(rng, E, *oracle.scale_shape(H, I))
    out = bf16_bits(bi8.moe_layer(bf16_to_dev(x), to_dev(logits), to_dev(w13), to_dev(ws13), to_dev(w2),
                                  to_dev(ws2), k, variant=variant))
    ref = oracle_moe_layer(x, logits, w13, ws13, w2, ws2, k)
    assert np.all(np.isfinite(bits_to_f64(out)))
    rel, frac_gt1, _ = gemm_report(out, ref)
    assert rel <= GEMM_REL_TOL, "moe layer: max rel err %.3e" % rel
    assert frac_gt1 <= 0.05, "moe layer: %.3f%% of outputs more than 1 ulp apart" % (100 * frac_gt1)
