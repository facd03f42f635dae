"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than its own formula: a
value the pages print, a closed form, an invariant, a special case that
reduces to a library routine (numpy integer/float64 matmul, torch's bf16
conversion), or brute force on tiny inputs.  Together they are chosen so that
a plausible mistake (dropped term, wrong sign or index, transposed operand,
wrong rounding) fails at least one of them.

Page cited: "[SGLang] Block-wise INT8: 블록 단위 정수 양자화" (blog.secrett2633.cloud).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(vals):
    return wl.to_bf16_bits(np.asarray(vals, np.float32))


def bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_bf16_of_f64(a):
    """Library rounding of float64 values that are exact in float32."""
    f = np.asarray(a, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(a, np.float64)), "not exact in fp32"
    return wl.to_bf16_bits(f)


def dequant_matmul(xq, xs, w, ws, bn, bk):
    """Brute force: dequantise both operands element-wise in fp64, then matmul."""
    M, K = xq.shape
    N = w.shape[0]
    kidx = np.arange(K) // bk
    nidx = np.arange(N) // bn
    xd = xq.astype(np.float64) * xs.astype(np.float64)[:, kidx]
    wd = w.astype(np.float64) * ws.astype(np.float64)[nidx][:, kidx]
    return xd @ wd.T


# ---------------------------------------------------------------- shapes --

def test_scale_shape_worked_example():
    """[BW8] §2 worked example (golden file)."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "scale_shapes.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for N, K, bn, bk, r, c in (map(int, row) for row in rows):
        assert oracle.scale_shape(N, K, bn, bk) == (r, c)


def test_scale_shape_partial_blocks_round_up():
    # A partial block still needs its own scale; one element past a block
    # boundary adds a row/column, an exact multiple does not.
    assert oracle.scale_shape(128, 128) == (1, 1)
    assert oracle.scale_shape(129, 128) == (2, 1)
    assert oracle.scale_shape(128, 129) == (1, 2)
    assert oracle.scale_shape(1, 1) == (1, 1)
    assert oracle.scale_shape(5000, 4000) == (40, 32)
    assert oracle.scale_shape(2 * 14336, 4096) == (224, 32)


def test_config_rules_golden():
    rules = dict(l.split() for l in open(os.path.join(GOLDEN, "config_rules.txt"))
                 if l.strip() and not l.startswith("#"))
    assert rules["weight_dtype"] == "int8" and rules["scale_dtype"] == "float32"
    assert int(rules["block_dims"]) == 2
    # the oracle's shape rule agrees with the default block
    bn, bk = int(rules["default_block_n"]), int(rules["default_block_k"])
    assert oracle.scale_shape(4096, 4096, bn, bk) == (32, 32)


# ------------------------------------------------------------------ bf16 --

@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80),
    (-2.5, 0xC020),
    (1.0 + 2.0 ** -8, 0x3F80),            # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie: a single rounding
    (2.0 ** -133, 0x0001),                # smallest subnormal
    (2.0 ** -134, 0x0000),                # tie between 0 and 2^-133 -> even (0)
    (1.5 * 2.0 ** -134, 0x0001),
    (2.0 ** -126, 0x0080),                # smallest normal
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie at the top -> even = inf
    (1e300, 0x7F80),
    (-0.0, 0x8000),
])
def test_f64_to_bf16_special_values(v, bits):
    assert oracle.f64_to_bf16(v) == bits


def test_f64_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(11)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),
                        (rng.standard_normal(2000) * 1e37).astype(np.float32)])
    ours = np.array([oracle.f64_to_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(ours, wl.to_bf16_bits(f))


def test_bf16_to_f32_exact():
    for b in (0x3F80, 0xC020, 0x0001, 0x7F7F, 0x8000):
        assert oracle.bf16_to_f32(b) == float(bits_to_f32([b])[0])


# ----------------------------------------------------------------- quant --

def test_quant_rne_ties():
    """A group whose amax is 127 has s = 1 exactly; halves round to even."""
    vals = [127.0, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5, -127.0, 0.0]
    x = bf16_bits([vals])
    xq, xs = oracle.quant_act(x, block_k=128)
    assert xs[0, 0] == 1.0
    assert xq[0].tolist() == [127, 0, 2, 2, -2, 126, 0, 4, -127, 0]   # half-away would give 1,3,-3,127


def test_quant_power_of_two_scales():
    # amax 254 -> s = 2;  amax 63.5 -> s = 0.5: quotients are exact.
    x = bf16_bits([[254.0, 3.0, -5.0, 1.0], [63.5, 0.25, -0.75, 1.25]])
    xq, xs = oracle.quant_act(x, block_k=4)
    assert xs[:, 0].tolist() == [2.0, 0.5]
    assert xq.tolist() == [[127, 2, -2, 0], [127, 0, -2, 2]]


def test_quant_division_reading_distinguishes_reciprocal():
    """q = rne(x / fl(amax/127)), not x * fl(127/amax) or x * fl(1/s).

    For amax = 1.484375 and x = -amax/2 the binary32 quotient x/s is exactly
    -63.5 (tie -> even -64) while both reciprocal forms land on -63.499996
    (-> -63).  Likewise amax = 6.96875, x = amax/2 gives 64 vs 63.  (Found by a
    float32 search; kept as a pin of the division reading.)"""
    x = bf16_bits([[1.484375, -0.7421875], [6.96875, 3.484375]])
    xq, xs = oracle.quant_act(x, block_k=2)
    assert xq[:, 1].tolist() == [-64, 64]


def test_quant_zero_group():
    x = np.zeros((2, 256), np.uint16)
    x[1, 200] = bf16_bits([3.0])[0]
    xq, xs = oracle.quant_act(x, block_k=128)
    assert xs.tolist() == [[0.0, 0.0], [0.0, np.float32(3.0) / np.float32(127.0)]]
    assert not xq[0].any()
    assert xq[1, 200] == 127 and np.count_nonzero(xq[1]) == 1


def test_quant_subnormal_group_keeps_denormals():
    # bf16 subnormals: the scale is a binary32 subnormal, not flushed to zero.
    b = np.array([[0x0001, 0x0003, 0x8002, 0x007F]], np.uint16)   # 1,3,-2,127 x 2^-133
    xq, xs = oracle.quant_act(b, block_k=4)
    s = xs[0, 0]
    assert 0 < s < np.finfo(np.float32).tiny
    assert s == np.float32(127 * 2.0 ** -133) / np.float32(127)
    assert xq[0].tolist() == [1, 3, -2, 127]


@pytest.mark.parametrize("outliers", [0.0, 0.01])
def test_quant_invariants_random(outliers):
    rng = np.random.default_rng(3)
    M, K, bk = 37, 1000, 128
    x = wl.activations(rng, M, K, outliers, 20.0)
    xq, xs = oracle.quant_act(x, block_k=bk)
    xf = bits_to_f32(x).astype(np.float64)
    KB = xs.shape[1]
    assert KB == 8 and xq.shape == (M, K)
    assert np.abs(xq.astype(np.int32)).max() <= 127
    for g in range(KB):
        blk = xf[:, g * bk:(g + 1) * bk]
        amax = np.abs(blk).max(axis=1)
        s = xs[:, g].astype(np.float64)
        # scale is amax/127 to within one binary32 rounding
        assert np.all(np.abs(s * 127 - amax) <= amax * 2.0 ** -23)
        q = xq[:, g * bk:(g + 1) * bk].astype(np.float64)
        # the amax element maps to +-127
        j = np.abs(blk).argmax(axis=1)
        assert np.all(np.abs(q[np.arange(M), j]) == 127)
        # reconstruction error within half a step (plus binary32 slack)
        err = np.abs(blk - q * s[:, None])
        assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -16))
        # sign and order are preserved
        assert np.all(np.sign(q) * np.sign(blk) >= 0)


def test_quant_outlier_isolation_and_group_independence():
    """[BW8] per-tensor vs per-block table: an outlier only affects its own block."""
    rng = np.random.default_rng(4)
    M, K = 6, 640
    x = wl.activations(rng, M, K)
    xq0, xs0 = oracle.quant_act(x)
    xf = bits_to_f32(x).copy()
    xf[2, 256:384] *= 20.0                 # one group of one token
    xq1, xs1 = oracle.quant_act(wl.to_bf16_bits(xf))
    changed = np.zeros_like(xs0, bool)
    changed[2, 2] = True
    assert np.array_equal(xs0[~changed], xs1[~changed])
    assert xs1[2, 2] > xs0[2, 2] * 10
    mask = np.ones_like(xq0, bool)
    mask[2, 256:384] = False
    assert np.array_equal(xq0[mask], xq1[mask])


def test_quant_ragged_and_padded_row_stride():
    rng = np.random.default_rng(5)
    M, K, ldx = 5, 200, 264
    x = wl.activations(rng, M, ldx)
    x[:, K:] = bf16_bits([1e30])[0]       # padding columns must be ignored
    xq, xs = oracle.quant_act(x, block_k=128, K=K)
    assert xq.shape == (M, K) and xs.shape == (M, 2)
    xq2, xs2 = oracle.quant_act(np.ascontiguousarray(x[:, :K]), block_k=128)
    assert np.array_equal(xq, xq2) and np.array_equal(xs, xs2)
    # the last group has 72 entries: its amax element is still +-127
    assert np.abs(xq[:, 128:].astype(int)).max(axis=1).tolist() == [127] * M


def test_quant_sign_symmetry():
    rng = np.random.default_rng(6)
    x = wl.activations(rng, 4, 384)
    xq, xs = oracle.quant_act(x)
    xqn, xsn = oracle.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(xs, xsn) and np.array_equal(xqn, -xq)


def test_quant_gather_commutes():
    """Quantisation is per token: quant(gather(x)) == gather(quant(x))."""
    rng = np.random.default_rng(7)
    x = wl.activations(rng, 50, 512)
    idx = rng.integers(0, 50, 120)
    xq, xs = oracle.quant_act(x)
    gq, gs = oracle.quant_act(x[idx])
    assert np.array_equal(gq, xq[idx]) and np.array_equal(gs, xs[idx])


def test_quant_rejects_non_finite():
    x = bf16_bits([[1.0, np.inf]])
    with pytest.raises(ValueError):
        oracle.quant_act(x)


# ------------------------------------------------------------------ gemm --

def test_gemm_integer_closed_form():
    """Unit scales: y is bf16(int64 matmul) exactly (sums < 2^24, exact in fp32)."""
    rng = np.random.default_rng(8)
    M, N, K = 9, 70, 1000
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs = np.ones((M, 8), np.float32)
    ws = np.ones((1, 8), np.float32)
    exact = xq.astype(np.int64) @ w.astype(np.int64).T
    y = oracle.gemm(xq, xs, w, ws)
    assert np.array_equal(y, torch_bf16_of_f64(exact))


def test_gemm_integer_pipeline_through_quant():
    """Integer activations with +-127 in every group quantise to themselves (s = 1)."""
    rng = np.random.default_rng(9)
    M, N, K = 4, 33, 384
    xi = rng.integers(-126, 127, (M, K)).astype(np.float32)
    xi[:, ::128] = 127.0
    xq, xs = oracle.quant_act(wl.to_bf16_bits(xi))
    assert np.all(xs == 1.0) and np.array_equal(xq.astype(np.float32), xi)
    w = wl.weights(rng, N, K)
    y = oracle.gemm(xq, xs, w, np.ones((1, 3), np.float32))
    assert np.array_equal(y, torch_bf16_of_f64(xi.astype(np.int64) @ w.astype(np.int64).T))


def test_gemm_power_of_two_scales_exact():
    """Power-of-two scales: every product and partial sum is exact even in fp32.

    |xq| <= 31 keeps each block sum below 2^19; scale products span 2^-14..2^-12,
    so any partial sum over the 5 blocks is a multiple of 2^-14 below 2^10 --
    fewer than 24 significant bits, exact in any summation order."""
    rng = np.random.default_rng(10)
    M, N, K, bn, bk = 7, 300, 520, 128, 128
    NB, KB = oracle.scale_shape(N, K, bn, bk)
    xq = rng.integers(-31, 32, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs = np.exp2(rng.integers(-8, -6, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(-6, -4, (NB, KB))).astype(np.float32)
    exact = dequant_matmul(xq, xs, w, ws, bn, bk)   # exact in float64 and float32
    assert np.array_equal(oracle.gemm(xq, xs, w, ws), torch_bf16_of_f64(exact))


@pytest.mark.parametrize("M,N,K,bn,bk", [
    (3, 5, 7, 2, 3), (16, 256, 256, 128, 128), (5, 300, 200, 128, 128),
    (11, 129, 257, 128, 128), (4, 64, 96, 16, 32), (2, 40, 50, 64, 8),
])
def test_gemm_brute_force_fp64(M, N, K, bn, bk):
    """Non-square, non-uniform scales: a swapped index or dropped factor fails."""
    rng = np.random.default_rng(M * 1000 + N)
    NB, KB = oracle.scale_shape(N, K, bn, bk)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs = wl.weight_scales(rng, M, KB)
    ws = wl.weight_scales(rng, NB, KB)
    ref = dequant_matmul(xq, xs, w, ws, bn, bk)
    y64 = oracle.gemm_f64(xq, xs, w, ws, block=(bn, bk))
    scale = np.abs(ref).max()
    assert np.abs(y64 - ref).max() <= 1e-12 * scale
    y16 = oracle.gemm(xq, xs, w, ws, block=(bn, bk))
    ref16 = np.array([oracle.f64_to_bf16(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    assert np.mean(y16 == ref16) > 0.999
    assert np.abs(bits_to_f32(y16).astype(np.float64) - ref).max() <= 2.0 ** -8 * scale


def test_gemm_bias_added_before_rounding():
    rng = np.random.default_rng(12)
    M, N, K = 3, 20, 128
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs, ws = np.ones((M, 1), np.float32), np.ones((1, 1), np.float32)
    bias_i = rng.integers(-1000, 1000, N).astype(np.float32)
    y = oracle.gemm(xq, xs, w, ws, bias=wl.to_bf16_bits(bias_i))
    exact = xq.astype(np.int64) @ w.astype(np.int64).T + bias_i.astype(np.int64)
    assert np.array_equal(y, torch_bf16_of_f64(exact))


def test_gemm_ragged_equals_zero_padded():
    """Zero padding K and N to whole blocks changes neither scales nor sums."""
    rng = np.random.default_rng(13)
    M, N, K = 6, 300, 200
    x = wl.activations(rng, M, K)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, 3, 2)
    xq, xs = oracle.quant_act(x)
    y = oracle.gemm(xq, xs, w, ws)
    xp = np.zeros((M, 256), np.uint16)
    xp[:, :K] = x
    wp = np.zeros((384, 256), np.int8)
    wp[:N, :K] = w
    xqp, xsp = oracle.quant_act(xp)
    assert np.array_equal(xsp, xs)
    yp = oracle.gemm(xqp, xsp, wp, ws)
    assert np.array_equal(yp[:M, :N], y)


def test_gemm_per_channel_degenerate_block():
    """block_n = 1, block_k = K: per-channel weights, per-token activations.

    Then y = (xq . w^T) * xs[m] * ws[n], a closed form."""
    rng = np.random.default_rng(14)
    M, N, K = 5, 17, 300
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs = wl.weight_scales(rng, M, 1)
    ws = wl.weight_scales(rng, N, 1)
    ref = (xq.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64) \
        * xs.astype(np.float64) * ws.astype(np.float64).T
    y64 = oracle.gemm_f64(xq, xs, w, ws, block=(1, K))
    assert np.abs(y64 - ref).max() <= 1e-13 * np.abs(ref).max()


def test_gemm_empty():
    y = oracle.gemm(np.zeros((0, 128), np.int8), np.zeros((0, 1), np.float32),
                    np.zeros((4, 128), np.int8), np.ones((1, 1), np.float32))
    assert y.shape == (0, 4)


# ------------------------------------------------------------------- moe --

def test_moe_single_expert_equals_gemm():
    rng = np.random.default_rng(15)
    R, N, K = 40, 130, 256
    x = wl.activations(rng, R, K)
    xq, xs = oracle.quant_act(x)
    w = wl.weights(rng, 1, N, K)
    ws = wl.weight_scales(rng, 1, 2, 2)
    y = oracle.moe_gemm(xq, xs, np.array([0, R], np.int32), w, ws)
    assert np.array_equal(y, oracle.gemm(xq, xs, w[0], ws[0]))


def test_moe_segments_brute_force_with_empty_experts():
    rng = np.random.default_rng(16)
    E, N, K = 5, 96, 200
    counts = np.array([7, 0, 13, 1, 0])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    xq = rng.integers(-127, 128, (R, K), dtype=np.int8)
    xs = wl.weight_scales(rng, R, 2)
    w = wl.weights(rng, E, N, K)
    ws = wl.weight_scales(rng, E, 1, 2)
    y = oracle.moe_gemm(xq, xs, off, w, ws)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if a == b:
            continue
        ref = dequant_matmul(xq[a:b], xs[a:b], w[e], ws[e], 128, 128)
        ref16 = np.array([oracle.f64_to_bf16(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
        assert np.mean(y[a:b] == ref16) > 0.99
        assert np.abs(bits_to_f32(y[a:b]) - ref).max() <= 2.0 ** -8 * np.abs(ref).max()


def test_moe_rejects_bad_offsets():
    xq = np.zeros((4, 128), np.int8)
    xs = np.zeros((4, 1), np.float32)
    w = np.zeros((2, 8, 128), np.int8)
    ws = np.ones((2, 1, 1), np.float32)
    for off in ([0, 3, 2], [1, 2, 4], [0, 2, 3]):
        with pytest.raises(ValueError):
            oracle.moe_gemm(xq, xs, np.array(off, np.int32), w, ws)


# ------------------------------------------------------- MoE steps (O3) --

def test_topk_two_experts_is_the_logistic_function():
    """E = 2, k = 1: the chosen weight is sigmoid(l_chosen - l_other) (scipy's expit)."""
    from scipy.special import expit
    rng = np.random.default_rng(21)
    lg = (rng.standard_normal((200, 2)) * 3).astype(np.float32)
    ids, w = oracle.topk_softmax(lg, 1)
    big = np.argmax(lg, axis=1)
    assert np.array_equal(ids[:, 0], big)
    d = lg[np.arange(200), big].astype(np.float64) - lg[np.arange(200), 1 - big].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], expit(d), rtol=1e-14)


def test_topk_matches_library_softmax_and_brute_force_order():
    from scipy.special import softmax
    rng = np.random.default_rng(22)
    lg = wl.router_logits(rng, 300, 8)
    for k in (1, 2, 3, 8):
        ids, w = oracle.topk_softmax(lg, k)
        p = softmax(lg.astype(np.float64), axis=1)
        for t in range(300):
            order = sorted(range(8), key=lambda e: (-p[t, e], e))[:k]
            assert list(ids[t]) == order
        np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)


def test_topk_ties_go_to_the_lower_expert_and_shift_invariance():
    lg = np.zeros((3, 8), np.float32)
    lg[1, [2, 5]] = 1.0            # two equal maxima
    lg[2] = [0, 3, 3, 3, 1, 1, 1, 1]
    ids, w = oracle.topk_softmax(lg, 2)
    assert ids.tolist() == [[0, 1], [2, 5], [1, 2]]
    np.testing.assert_allclose(w[0], [1 / 8, 1 / 8], rtol=1e-15)
    ids2, w2 = oracle.topk_softmax(lg + np.float32(50.0), 2)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-13)


def test_topk_renormalised_weights_sum_to_one():
    lg = wl.router_logits(np.random.default_rng(23), 100, 8)
    ids, w = oracle.topk_softmax(lg, 2, renorm=True)
    ids0, w0 = oracle.topk_softmax(lg, 2)
    assert np.array_equal(ids, ids0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(w / w0, np.repeat((1 / w0.sum(1))[:, None], 2, axis=1), rtol=1e-12)


def test_align_is_a_stable_sort_by_expert():
    """Brute force: Python's sort on the key (expert, token, slot)."""
    rng = np.random.default_rng(24)
    for T, E, k in [(64, 8, 2), (7, 3, 1), (33, 16, 4), (1, 4, 2)]:
        ids, _ = oracle.topk_softmax(wl.router_logits(rng, T, E), k)
        st, off, row_of = oracle.moe_align(ids, E)
        keys = sorted((int(ids[t, s]), t, s) for t in range(T) for s in range(k))
        assert st.tolist() == [t for _, t, _ in keys]
        counts = np.bincount(ids.ravel(), minlength=E)
        assert off.tolist() == [0] + np.cumsum(counts).tolist()
        for r, (e, t, s) in enumerate(keys):
            assert row_of[t, s] == r and off[e] <= r < off[e + 1]


def test_dispatch_layout_is_expert_sorted():
    rng = np.random.default_rng(17)
    logits = wl.router_logits(rng, 64, 8)
    ids, _ = oracle.topk_softmax(logits, 2)
    tok, off, _ = oracle.moe_align(ids, 8)
    assert off[0] == 0 and off[-1] == 128 and np.all(np.diff(off) >= 0)
    top2 = np.argsort(-logits, axis=1)[:, :2]
    for e in range(8):
        seg = tok[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) >= 0)
        assert all(e in top2[t] for t in seg)


def test_silu_mul_special_values_and_library_form():
    """silu(z) * 1 against z * expit(z) (scipy); silu(0) = 0; silu(z) - silu(-z) = z."""
    from scipy.special import expit
    z = np.array([0.0, 1.0, -1.0, 2.5, -2.5, 10.0, -10.0, 80.0, -80.0, 0.001, -30000.0], np.float32)
    zb = bf16_bits(z)
    h = np.concatenate([zb[None, :], bf16_bits(np.ones_like(z))[None, :]], axis=1)
    a = oracle.silu_mul(h)[0]
    zf = bits_to_f32(zb).astype(np.float64)
    ref = np.array([oracle.f64_to_bf16(v) for v in zf * expit(zf)], np.uint16)
    assert np.array_equal(a, ref)
    assert a[0] == 0 and bits_to_f32(a[1]) == bits_to_f32(bf16_bits([0.7310585786300049]))[0]
    # odd part: silu(z) - silu(-z) = z, to bf16 rounding
    for i in (1, 3, 5, 7):
        np.testing.assert_allclose(bits_to_f32(a[i]) - bits_to_f32(a[i + 1]), zf[i], rtol=2 ** -7)


def test_silu_mul_gate_up_order_and_scaling():
    """Column i of the output uses gate column i and up column I + i; up scales linearly."""
    rng = np.random.default_rng(25)
    R, I = 5, 40
    g = wl.activations(rng, R, I)
    u = wl.activations(rng, R, I)
    a = oracle.silu_mul(np.concatenate([g, u], axis=1))
    a_swapped = oracle.silu_mul(np.concatenate([u, g], axis=1))
    assert not np.array_equal(a, a_swapped)
    two = bf16_bits(np.full((R, I), 2.0, np.float32))
    a1 = oracle.silu_mul(np.concatenate([g, bf16_bits(np.ones((R, I), np.float32))], axis=1))
    a2 = oracle.silu_mul(np.concatenate([g, two], axis=1))
    assert np.array_equal(bits_to_f32(a2), 2 * bits_to_f32(a1))          # exact power-of-two scaling
    from scipy.special import expit
    gf = bits_to_f32(g).astype(np.float64)
    uf = bits_to_f32(u).astype(np.float64)
    np.testing.assert_allclose(bits_to_f32(a), gf * expit(gf) * uf, rtol=2 ** -8, atol=1e-30)


def test_combine_special_cases():
    rng = np.random.default_rng(26)
    T, k, H = 6, 2, 24
    ids, _ = oracle.topk_softmax(wl.router_logits(rng, T, 4), k)
    _, _, row_of = oracle.moe_align(ids, 4)
    y2 = wl.activations(rng, T * k, H)
    # k = 1 with unit weight: a pure gather
    out1 = oracle.combine(y2, row_of[:, :1], np.ones((T, 1), np.float32))
    assert np.array_equal(out1, y2[row_of[:, 0]])
    # equal rows and weights summing to one: the row itself
    y_eq = y2.copy()
    y_eq[row_of[:, 1]] = y_eq[row_of[:, 0]]
    w = np.tile(np.array([[0.25, 0.75]], np.float32), (T, 1))
    assert np.array_equal(oracle.combine(y_eq, row_of, w), y2[row_of[:, 0]])
    # slot weights swap with the slots
    w2 = rng.random((T, k)).astype(np.float32)
    swapped = oracle.combine(y2, row_of[:, ::-1], w2[:, ::-1])
    assert np.array_equal(swapped, oracle.combine(y2, row_of, w2))
    # doubling the weights doubles the output exactly
    assert np.array_equal(bits_to_f32(oracle.combine(y2, row_of, 2 * w2)),
                          2 * bits_to_f32(oracle.combine(y2, row_of, w2)))


# ------------------------------------------------ offline weight quantiser --

def test_quant_weight_block_rows_equal_activation_quantiser():
    """block_n = 1 is the per-(row, K-group) encoding of the activations."""
    rng = np.random.default_rng(31)
    w = wl.activations(rng, 37, 300, 0.02)
    wq, ws = oracle.quant_weight(w, block=(1, 128))
    xq, xs = oracle.quant_act(w)
    assert np.array_equal(wq, xq) and np.array_equal(ws, xs)


def test_quant_weight_scale_shape_and_ties():
    w = np.zeros((4096, 4096), np.uint16)
    wq, ws = oracle.quant_weight(w)
    assert ws.shape == (32, 32) and not ws.any() and not wq.any()          # the pages' worked example
    blk = np.zeros((128, 128), np.float32)
    blk[5, 7] = 127.0                                                      # s = 1 exactly
    blk[0, :5] = [0.5, 1.5, 2.5, -2.5, 126.5]
    blk[100, 3] = -127.0
    wq, ws = oracle.quant_weight(bf16_bits(blk))
    assert ws[0, 0] == 1.0
    assert wq[0, :5].tolist() == [0, 2, 2, -2, 126]                         # round half to even
    assert wq[5, 7] == 127 and wq[100, 3] == -127


def test_quant_weight_invariants_and_ragged_padding():
    rng = np.random.default_rng(32)
    N, K = 300, 400
    w = wl.activations(rng, N, K)
    wq, ws = oracle.quant_weight(w)
    assert ws.shape == (3, 4) and np.abs(wq.astype(int)).max() <= 127
    wf = bits_to_f32(w).astype(np.float64)
    s = np.repeat(np.repeat(ws, 128, 0), 128, 1)[:N, :K].astype(np.float64)
    assert np.all(np.abs(wf - wq * s) <= s * (0.5 + 2.0 ** -16))
    for bn in range(3):                                                   # each block's max hits 127
        for bk in range(4):
            blk = np.abs(wq[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128].astype(int))
            assert blk.max() == 127
    # zero padding to whole blocks changes nothing
    wp = np.zeros((384, 512), np.uint16)
    wp[:N, :K] = w
    wqp, wsp = oracle.quant_weight(wp)
    assert np.array_equal(wqp[:N, :K], wq) and np.array_equal(wsp, ws)


def test_quant_weight_transpose_swaps_blocks():
    rng = np.random.default_rng(33)
    w = wl.activations(rng, 200, 136)
    wq, ws = oracle.quant_weight(w, block=(64, 32))
    wqt, wst = oracle.quant_weight(np.ascontiguousarray(w.T), block=(32, 64))
    assert np.array_equal(wqt, wq.T) and np.array_equal(wst, ws.T)


def test_quant_weight_row_stride():
    rng = np.random.default_rng(34)
    w = wl.activations(rng, 50, 272)
    wq, ws = oracle.quant_weight(w, K=256)          # ldw = 272
    wq2, ws2 = oracle.quant_weight(np.ascontiguousarray(w[:, :256]))
    assert np.array_equal(wq, wq2) and np.array_equal(ws, ws2)
