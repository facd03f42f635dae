"""Parity of the HIP path with the CPU oracle, element by element.

Quantisation (codes and scales) must match bit-exactly; GEMM outputs must be
within max-relative error 1e-2 of the output magnitude (``GEMM_REL_TOL``).
Integer-valued and power-of-two cases, whose fp32 sums are exact in any
order, must match bit-exactly.  At the full workload sizes, the oracle
computes sampled rows (all N columns of each sampled row), and the GPU runs in
the same launch configuration the benchmark times (the library picks the
kernel from the shape).

Page cited: "[SGLang] Block-wise INT8: 블록 단위 정수 양자화" (blog.secrett2633.cloud).
"""
import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import oracle
import workloads as wl
from gpu_util import (assert_gemm_close, bf16_bits, bf16_to_dev, bits_to_f64, device,
                      oracle_gemm_rows, to_dev)

pytestmark = pytest.mark.gpu


def gpu_quant(x_bits):
    xq, xs = bi8.quant_act(bf16_to_dev(x_bits))
    return xq.cpu().numpy(), xs.cpu().numpy()


def make_case(seed, M, N, K, outlier_frac=0.0):
    rng = wl.rng_for(seed)
    x = wl.activations(rng, M, K, outlier_frac)
    w = wl.weights(rng, N, K)
    NB, KB = oracle.scale_shape(N, K)
    ws = wl.weight_scales(rng, NB, KB)
    return x, w, ws


def sample_rows(M, n, rng):
    """Rows spread over the whole range, always including the first and last."""
    if M <= n:
        return np.arange(M)
    inner = rng.choice(np.arange(1, M - 1), n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], inner]))


# activation rows per workgroup tile of each kernel (the skinny kernel takes
# every row of the problem in one tile column)
TILE_M = {bi8.GEMM_SKINNY: 64, bi8.GEMM_TILE_128X64: 64, bi8.GEMM_TILE_256X128: 128,
          bi8.GEMM_TILE_256X256: 256}


def tile_rows(start, stop, bm, rng, per_tile=1):
    """Rows of [start, stop) covering every bm-row tile that starts at `start`:
    `per_tile` rows drawn inside each tile, plus the first and the last row."""
    rows = {start, stop - 1}
    for t0 in range(start, stop, bm):
        t1 = min(stop, t0 + bm)
        rows.update(int(r) for r in rng.choice(np.arange(t0, t1), min(per_tile, t1 - t0), replace=False))
    return np.array(sorted(rows))


# ------------------------------------------------------------------ quant --

@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "ragged", "down"])
def test_quant_bit_exact_workloads(name):
    c = wl.CONFIGS[name]
    x = wl.activations(wl.rng_for(c["seed"]), c["M"], c["K"], c.get("outlier_frac", 0.0))
    q_ref, s_ref = oracle.quant_act(x)
    q, s = gpu_quant(x)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


def test_quant_special_values_bit_exact():
    rows = []
    rows.append([127.0, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5] + [0.0] * 120)   # RNE ties, s = 1
    rows.append([0.0] * 128)                                                     # zero group
    rows.append([1.484375, -0.7421875] + [0.0] * 126)                            # x/s == -63.5 tie
    rows.append([6.96875, 3.484375] + [0.0] * 126)
    x = wl.to_bf16_bits(np.array(rows, np.float32))
    sub = np.zeros((1, 128), np.uint16)
    sub[0, :4] = [0x0001, 0x0003, 0x8002, 0x007F]                                # subnormal group
    x = np.concatenate([x, sub])
    q_ref, s_ref = oracle.quant_act(x)
    q, s = gpu_quant(x)
    assert np.array_equal(q, q_ref) and np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert q[0, :8].tolist() == [127, 0, 2, 2, -2, 126, 0, 4]
    assert s[1, 0] == 0.0 and not q[1].any()
    assert 0 < s[4, 0] < np.finfo(np.float32).tiny


def groups_below(amax_bits):
    """Every bf16 value of magnitude <= amax, 127 per group with amax itself first."""
    b = np.arange(0, 0x7F80, dtype=np.uint32)          # every finite non-negative bf16
    vals = b[b <= amax_bits]
    vals = np.concatenate([vals, vals | 0x8000]).astype(np.uint16)
    n = -(-len(vals) // 127)
    x = np.zeros((n, 128), np.uint16)
    x[:, 0] = amax_bits
    flat = x[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(n, 127)
    return x


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4040, 0x42C8, 0x42FE, 0x3E9A, 0x0380, 0x0001, 0x7F7F])
def test_quant_every_bf16_below_amax_bit_exact(amax_bits):
    """Covers each quotient x / s the group can produce, ties and near-ties included
    (amax 1, 3, 100, 127, 0.3, 2^-120, the smallest subnormal, the largest finite)."""
    x = groups_below(amax_bits)
    q_ref, s_ref = oracle.quant_act(x)
    q, s = gpu_quant(x)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_quant_every_bf16_for_every_mantissa_of_amax_bit_exact():
    """The codes are multiplies by the hardware reciprocal of s (within 1 ulp),
    with the division wherever the product comes within 2^-14 of a half-integer.
    For normal values, scaling amax and x by a power of two scales s and every
    quotient exactly, so amax in [1, 2) at each of its 128 bf16 mantissas covers
    the normal range. The 127 subnormal maxima (s subnormal, reciprocal
    overflowing) and the 128 largest (smallest normal reciprocals) cover the
    ends. Every bf16 input of magnitude <= amax for each: ~13 M codes."""
    maxima = list(range(0x3F80, 0x4000)) + list(range(0x0001, 0x0080)) + list(range(0x7F00, 0x7F80))
    x = np.concatenate([groups_below(a) for a in maxima])
    q_ref, s_ref = oracle.quant_act(x)
    q, s = gpu_quant(x)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    bad = np.nonzero(np.any(q != q_ref, axis=1))[0]
    assert bad.size == 0, "groups with differing codes: %d (first amax bits %#06x)" % (bad.size, x[bad[0], 0])


@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (5, 144), (7, 4000), (64, 128), (2, 14336),
                                 (65537, 128)])
def test_quant_shapes_bit_exact(M, K):
    rng = np.random.default_rng(M * 7 + K)
    x = wl.activations(rng, M, K, 0.02)
    q_ref, s_ref = oracle.quant_act(x)
    q, s = gpu_quant(x)
    assert np.array_equal(q, q_ref) and np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


def test_quant_row_stride():
    rng = np.random.default_rng(21)
    M, K, ldx = 9, 384, 520
    full = wl.activations(rng, M, ldx)
    xd = bf16_to_dev(full)[:, :K]
    assert xd.stride(0) == ldx
    xq, xs = bi8.quant_act(xd)
    q_ref, s_ref = oracle.quant_act(full, K=K)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


# ------------------------------------------------------------------- gemm --

def run_gemm(xq, xs, w, ws, bias=None, variant=None):
    y = bi8.gemm(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws),
                 None if bias is None else bf16_to_dev(bias), variant=variant)
    return bf16_bits(y)


TILED = [bi8.GEMM_TILE_128X64, bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256]


SHAPES = [
    # skinny path
    (1, 16, 16), (1, 256, 256), (8, 4096, 512), (8, 100, 4000), (16, 300, 144), (17, 257, 1040),
    (32, 512, 384), (5, 1000, 4096), (32, 100, 2000), (31, 64, 2096), (3, 40, 21840),
    # more tokens (tiled, or skinny while N is small), ragged N / K / M
    (33, 256, 256), (64, 128, 128), (100, 1000, 272), (129, 384, 400), (333, 500, 4000),
    (256, 2048, 256), (300, 5000, 128), (200, 7, 128), (1000, 16, 64), (513, 1024, 1024),
    # skinny with 3 and 4 token tiles; few tokens on a wide N (tiled by choice)
    (40, 1000, 1040), (64, 520, 2064), (48, 300, 4000), (8, 28672, 256),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_shapes_vs_oracle(M, N, K):
    x, w, ws = make_case((M, N, K), M, N, K)
    xq, xs = oracle.quant_act(x)
    y_ref = oracle.gemm(xq, xs, w, ws)
    y = run_gemm(xq, xs, w, ws)
    assert_gemm_close(y, y_ref, "M=%d N=%d K=%d" % (M, N, K))
    variants = TILED + ([bi8.GEMM_SKINNY] if M <= 64 else [])
    for v in variants:
        assert_gemm_close(run_gemm(xq, xs, w, ws, variant=v), y_ref, "M=%d N=%d K=%d variant %d" % (M, N, K, v))


# Shapes spanning several tiles of every tiled kernel, with ragged M, N and K
# tails, including a tile row with a single valid activation row.  The 128 x 64
# kernel runs a 4-stage ring on grids of at most 256 tiles and a 3-stage ring
# on larger ones (the last two shapes: 336 and 342 tiles, with 25 and 11 K
# blocks, so both leave a partial turn of the ring).
@pytest.mark.parametrize("M,N,K", [(513, 520, 1040), (769, 1000, 400), (257, 2056, 272),
                                   (1000, 2600, 3088), (1100, 2400, 1296)])
def test_gemm_tiled_variants_multi_tile(M, N, K):
    x, w, ws = make_case((M, N, K, 7), M, N, K)
    xq, xs = oracle.quant_act(x)
    y_ref = oracle.gemm(xq, xs, w, ws)
    for v in TILED:
        assert_gemm_close(run_gemm(xq, xs, w, ws, variant=v), y_ref, "M=%d N=%d K=%d variant %d" % (M, N, K, v))


@pytest.mark.parametrize("name", ["tiny", "decode", "ragged", "prefill", "gate_up", "down"])
def test_gemm_workloads_vs_oracle(name):
    """Full-size workloads in the kernel the library picks: rows sampled in every
    m-tile of that kernel (all N columns of each), the whole output finite."""
    c = wl.CONFIGS[name]
    M, N, K = c["M"], c["N"], c["K"]
    x, w, ws = make_case(c["seed"], M, N, K, c.get("outlier_frac", 0.0))
    xq_d, xs_d = bi8.quant_act(bf16_to_dev(x))
    y = bf16_bits(bi8.gemm(xq_d, xs_d, to_dev(w), to_dev(ws)))
    xq, xs = xq_d.cpu().numpy(), xs_d.cpu().numpy()
    bm = TILE_M[bi8.gemm_select(M, N, K)]
    rows = tile_rows(0, M, bm, np.random.default_rng(5), per_tile=2 if N * K <= 2 ** 26 else 1)
    assert len(rows) >= min(M, -(-M // bm))
    q_ref, s_ref = oracle.quant_act(x[rows])
    assert np.array_equal(xq[rows], q_ref) and np.array_equal(xs[rows], s_ref)
    y_ref = oracle_gemm_rows(q_ref, s_ref, w, ws)
    assert_gemm_close(y[rows], y_ref, name)
    assert np.all(np.isfinite(bits_to_f64(y))), name + ": non-finite output"


@pytest.mark.parametrize("M,N,K", [(8, 512, 1024), (24, 300, 1040), (200, 520, 1024), (333, 260, 896)])
def test_gemm_integer_closed_form_bit_exact(M, N, K):
    """Unit scales and integer activations: y == bf16(int64 matmul) exactly."""
    rng = np.random.default_rng(M + N + K)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    NB, KB = oracle.scale_shape(N, K)
    xs = np.ones((M, KB), np.float32)
    ws = np.ones((NB, KB), np.float32)
    exact = (xq.astype(np.int64) @ w.astype(np.int64).T).astype(np.float32)
    y = run_gemm(xq, xs, w, ws)
    assert np.array_equal(y, wl.to_bf16_bits(exact))


@pytest.mark.parametrize("K", [16, 48, 144, 400, 1040, 1296, 2000, 4000, 4080])
@pytest.mark.parametrize("offset", [0, 16, 48, 80])
def test_gemm_rows_off_the_line_bit_exact(K, offset):
    """Rows that do not start on a 128-byte line (K % 128 != 0, or operands at
    a 16-byte offset from a line) through the small-grid kernel the library
    picks and the forced 128 x 64 variant.  Unit scales and int8 activations:
    y == bf16(int64 matmul) exactly, for every alignment of the rows, with a K
    tail in the last block and several tiles."""
    M, N = 200, 1000
    rng = np.random.default_rng(K * 131 + offset)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    NB, KB = oracle.scale_shape(N, K)
    exact = (xq.astype(np.int64) @ w.astype(np.int64).T)
    assert np.abs(exact).max() < 2 ** 24   # every fp32 partial sum exact
    dev = device()
    xbuf = torch.zeros(offset + M * K + 256, dtype=torch.int8, device=dev)
    wbuf = torch.zeros(offset + N * K + 256, dtype=torch.int8, device=dev)
    xq_d = xbuf[offset:offset + M * K].view(M, K)
    w_d = wbuf[offset:offset + N * K].view(N, K)
    xq_d.copy_(torch.from_numpy(xq))
    w_d.copy_(torch.from_numpy(w))
    xs = torch.ones((M, KB), dtype=torch.float32, device=dev)
    ws = torch.ones((NB, KB), dtype=torch.float32, device=dev)
    for v in (None, bi8.GEMM_TILE_128X64):
        y = bf16_bits(bi8.gemm(xq_d, xs, w_d, ws, variant=v))
        assert np.array_equal(y, wl.to_bf16_bits(exact.astype(np.float32))), "K=%d offset=%d variant %s" % (
            K, offset, v)


@pytest.mark.parametrize("M,N,K", [(7, 300, 528), (150, 600, 528)])
def test_gemm_power_of_two_bit_exact(M, N, K):
    """Power-of-two scales, |xq| <= 31: every partial sum exact in fp32.

    5 K blocks (the last 16 wide); block sums < 2^19, scale products within a
    factor 4, so every partial sum has fewer than 24 significant bits."""
    rng = np.random.default_rng(10 + M)
    NB, KB = oracle.scale_shape(N, K)
    xq = rng.integers(-31, 32, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs = np.exp2(rng.integers(-8, -6, (M, KB))).astype(np.float32)
    ws = np.exp2(rng.integers(-6, -4, (NB, KB))).astype(np.float32)
    y = run_gemm(xq, xs, w, ws)
    assert np.array_equal(y, oracle.gemm(xq, xs, w, ws))


@pytest.mark.parametrize("variant", [bi8.GEMM_SKINNY] + TILED)
def test_gemm_subnormal_outputs_bit_exact(variant):
    """Outputs in the fp32 and bf16 subnormal range, through every kernel: with
    activation scales 2^-75 or 2^-76 and weight scales 2^-70, every product
    and partial sum is a multiple of 2^-146 below 2^-123 (at most 23
    significant bits), so the fp32 sums are exact in any order and the only
    rounding is the one to bf16 (subnormals kept, ties to even)."""
    rng = np.random.default_rng(77)
    M, N, K = 40, 300, 528
    NB, KB = oracle.scale_shape(N, K)
    xq = rng.integers(-31, 32, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    xs = np.exp2(rng.choice([-75, -76], (M, KB))).astype(np.float32)
    ws = np.full((NB, KB), 2.0 ** -70, np.float32)
    ref = oracle.gemm(xq, xs, w, ws)
    assert np.mean((ref & 0x7F80) == 0) > 0.3, "the case must reach bf16 subnormals"
    assert np.array_equal(run_gemm(xq, xs, w, ws, variant=variant), ref)


@pytest.mark.parametrize("M", [4, 96])
def test_gemm_bias(M):
    N, K = 384, 256
    x, w, ws = make_case(99 + M, M, N, K)
    bias = wl.activations(np.random.default_rng(1), 1, N)[0]
    xq, xs = oracle.quant_act(x)
    y = run_gemm(xq, xs, w, ws, bias)
    assert_gemm_close(y, oracle.gemm(xq, xs, w, ws, bias=bias), "bias")


def test_linear_pipeline_matches_oracle():
    M, N, K = 40, 640, 768
    x, w, ws = make_case(31, M, N, K, 0.01)
    y = bf16_bits(bi8.linear(bf16_to_dev(x), to_dev(w), to_dev(ws)))
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(y, oracle.gemm(xq, xs, w, ws), "linear")


@pytest.mark.parametrize("M,N,K,ldx", [
    (1, 256, 256, 256), (5, 300, 4000, 4000), (16, 1000, 1040, 1048), (33, 512, 144, 152),
    (200, 384, 1040, 1040),
])
def test_linear_equals_quant_then_gemm(M, N, K, ldx):
    """One C call, bit-identical to quant_act + gemm, and within tolerance of
    the oracle; x with a row stride, with and without bias."""
    x, w, ws = make_case((M, N, K, 3), M, N, K, 0.01)
    xd = torch.zeros((M, ldx), dtype=torch.bfloat16, device=device())
    xd[:, :K] = bf16_to_dev(x)
    wd, wsd = to_dev(w), to_dev(ws)
    bias = wl.activations(np.random.default_rng(M), 1, N)[0]
    for b in (None, bias):
        bd = None if b is None else bf16_to_dev(b)
        y_one = bf16_bits(bi8.linear(xd[:, :K], wd, wsd, bias=bd))
        xq, xs = bi8.quant_act(xd[:, :K])
        y_two = bf16_bits(bi8.gemm(xq, xs, wd, wsd, bias=bd))
        assert np.array_equal(y_one, y_two)
        q_ref, s_ref = oracle.quant_act(x)
        assert_gemm_close(y_one, oracle.gemm(q_ref, s_ref, w, ws, bias=b), "linear M=%d" % M)


@pytest.fixture(scope="module")
def max_k_case():
    """K = 2^23, the largest K the C ABI accepts: a 256-row weight tile is then
    exactly 2^31 bytes, the largest buffer range a kernel addresses."""
    M, N, K = 40, 256, 1 << 23
    rng = wl.rng_for((1 << 23, 1))
    x = wl.activations(rng, M, K)
    w = wl.weights(rng, N, K)
    ws = wl.weight_scales(rng, *oracle.scale_shape(N, K))
    xq, xs = bi8.quant_act(bf16_to_dev(x))
    yield x, w, ws, xq, xs, to_dev(w), to_dev(ws)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant,rows", [
    (bi8.GEMM_SKINNY, 8), (bi8.GEMM_TILE_128X64, 40), (bi8.GEMM_TILE_256X128, 40), (bi8.GEMM_TILE_256X256, 40),
])
def test_gemm_at_max_k_every_kernel(max_k_case, variant, rows):
    x, w, ws, xq, xs, wd, wsd = max_k_case
    y = bf16_bits(bi8.gemm(xq[:rows], xs[:rows], wd, wsd, variant=variant))
    q_ref, s_ref = oracle.quant_act(x[rows - 1:rows])
    # the codes of the sampled row are bit-exact, and its outputs within tolerance
    assert np.array_equal(xq[rows - 1:rows].cpu().numpy(), q_ref)
    assert np.array_equal(xs[rows - 1:rows].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert_gemm_close(y[rows - 1:rows], oracle.gemm(q_ref, s_ref, w, ws), "K = 2^23, variant %d" % variant)


def test_linear_workspaces_hold_the_codes():
    """Caller-given workspaces hold the quantised activations on return."""
    M, N, K = 8, 512, 1040
    x, w, ws = make_case(77, M, N, K)
    KB = (K + 127) // 128
    xq = torch.empty((M, K), dtype=torch.int8, device=device())
    xs = torch.empty((M, KB), dtype=torch.float32, device=device())
    wd, wsd = to_dev(w), to_dev(ws)
    y = bi8.linear(bf16_to_dev(x), wd, wsd, xq=xq, xs=xs)
    q_ref, s_ref = oracle.quant_act(x)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert_gemm_close(bf16_bits(y), oracle.gemm(q_ref, s_ref, w, ws), "linear with workspaces")
    with pytest.raises(ValueError):
        bi8.linear(bf16_to_dev(x), wd, wsd, xq=xq[:, :16])
    with pytest.raises(ValueError):
        bi8.linear(bf16_to_dev(x), wd, wsd, xs=xs[:, :2])


def test_gemm_unaligned_output_rows():
    """N % 4 != 0 takes the element-wise store path."""
    M, N, K = 70, 333, 256
    x, w, ws = make_case(41, M, N, K)
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(run_gemm(xq, xs, w, ws), oracle.gemm(xq, xs, w, ws), "N=333")


def test_gemm_empty_and_errors():
    dev = device()
    xq = torch.zeros((0, 128), dtype=torch.int8, device=dev)
    xs = torch.zeros((0, 1), dtype=torch.float32, device=dev)
    w = torch.zeros((8, 128), dtype=torch.int8, device=dev)
    ws = torch.ones((1, 1), dtype=torch.float32, device=dev)
    assert bi8.gemm(xq, xs, w, ws).shape == (0, 8)
    with pytest.raises(bi8.BlockInt8Error, match="BI8_ERR_BLOCK"):
        bi8.gemm(xq, xs, w, ws, block=(64, 128))


# -------------------------------------------------------------------- moe --

MOE_VARIANTS = [None, bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256]


def moe_case(seed, counts, N, K):
    rng = np.random.default_rng(seed)
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    x = wl.activations(rng, R, K)
    w = wl.weights(rng, E, N, K)
    NB, KB = oracle.scale_shape(N, K)
    ws = wl.weight_scales(rng, E, NB, KB)
    return x, off, w, ws


@pytest.mark.parametrize("counts,N,K", [
    ([40], 256, 256),
    ([7, 0, 130, 1, 0, 257], 300, 400),
    ([0, 0, 128], 128, 128),
    ([300, 5, 33, 128, 129], 512, 1024),
    # experts longer than one tile group (16 m-tiles): 33 and 17 tiles of 128
    # rows, 17 and 9 of 256, so a group boundary falls inside an expert
    ([4200, 0, 2100, 3], 512, 256),
])
@pytest.mark.parametrize("variant", MOE_VARIANTS)
def test_moe_small_vs_oracle(counts, N, K, variant):
    x, off, w, ws = moe_case(len(counts) * 100 + N, counts, N, K)
    xq, xs = oracle.quant_act(x)
    y_ref = oracle.moe_gemm(xq, xs, off, w, ws)
    y = bf16_bits(bi8.moe_gemm(to_dev(xq), to_dev(xs), to_dev(off), to_dev(w), to_dev(ws),
                               variant=variant))
    assert_gemm_close(y, y_ref, "moe %s variant %s" % (counts, variant))


@pytest.mark.parametrize("variant", [bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256])
def test_moe_one_expert_equals_dense_gemm(variant):
    x, off, w, ws = moe_case(7, [500], 640, 512)
    xq, xs = to_dev(oracle.quant_act(x)[0]), to_dev(oracle.quant_act(x)[1])
    y_moe = bf16_bits(bi8.moe_gemm(xq, xs, to_dev(off), to_dev(w), to_dev(ws), variant=variant))
    y_dense = bf16_bits(bi8.gemm(xq, xs, to_dev(w[0]), to_dev(ws[0]), variant=variant))
    assert np.array_equal(y_moe, y_dense)


# ------------------------------------------------------------- split K --
#
# blockint8_gemm_ws splits K between workgroups on grids of few 128 x 64 tiles
# with small outputs (fp32 partial sums in the caller workspace, added in
# split order by a second launch).  The shapes below all split (asserted
# through the workspace size); larger outputs do not.

SPLIT_SHAPES = [(129, 1000, 3088), (257, 2056, 4000), (64, 8192, 4096), (100, 6000, 8192), (150, 1001, 2048)]


def ws_bytes(M, N, K):
    return bi8.gemm_workspace_size(M, N, K)


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_gemm_ws_split_k_vs_oracle(M, N, K):
    nws = ws_bytes(M, N, K)
    assert nws >= 2 * 4 * M * N, "the shape must split K"
    x, w, ws = make_case((M, N, K, 21), M, N, K)
    xq, xs = oracle.quant_act(x)
    wsp = torch.full((nws,), 0xFF, dtype=torch.uint8, device=device())   # garbage: needs no initialisation
    args = (to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws))
    y = bf16_bits(bi8.gemm_ws(*args, wsp))
    rows = tile_rows(0, M, 64, np.random.default_rng(M), per_tile=2)
    assert_gemm_close(y[rows], oracle_gemm_rows(xq[rows], xs[rows], w, ws), "split K %dx%dx%d" % (M, N, K))
    assert np.all(np.isfinite(bits_to_f64(y)))
    # deterministic, and within the tolerance of the unsplit kernel everywhere
    assert np.array_equal(bf16_bits(bi8.gemm_ws(*args, wsp)), y)
    assert_gemm_close(y, bf16_bits(bi8.gemm(*args)), "split vs unsplit")


def test_gemm_ws_split_k_integer_bit_exact():
    """Unit scales, |xq| <= 31: every partial sum is an integer below 2^24, so
    the split sums are exact in any order: y == bf16(int64 matmul)."""
    M, N, K = 200, 512, 2048
    assert ws_bytes(M, N, K) > 0
    rng = np.random.default_rng(4)
    xq = rng.integers(-31, 32, (M, K), dtype=np.int8)
    w = wl.weights(rng, N, K)
    NB, KB = oracle.scale_shape(N, K)
    wsp = torch.empty((ws_bytes(M, N, K),), dtype=torch.uint8, device=device())
    y = bf16_bits(bi8.gemm_ws(to_dev(xq), to_dev(np.ones((M, KB), np.float32)), to_dev(w),
                              to_dev(np.ones((NB, KB), np.float32)), wsp))
    exact = (xq.astype(np.int64) @ w.astype(np.int64).T).astype(np.float32)
    assert np.array_equal(y, wl.to_bf16_bits(exact))


def test_gemm_ws_bias_odd_n_and_unaligned_y():
    M, N, K = 150, 1001, 2048
    nws = ws_bytes(M, N, K)
    assert nws > 0
    x, w, ws = make_case(5, M, N, K)
    bias = wl.activations(np.random.default_rng(6), 1, N)[0]
    xq, xs = oracle.quant_act(x)
    wsp = torch.empty((nws,), dtype=torch.uint8, device=device())
    ybuf = torch.zeros((M * N + 1,), dtype=torch.bfloat16, device=device())
    y = ybuf[1:].view(M, N)    # 2-byte aligned rows, element-wise stores
    bi8.gemm_ws(to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws), wsp, bias=bf16_to_dev(bias), y=y)
    assert_gemm_close(bf16_bits(y), oracle.gemm(xq, xs, w, ws, bias=bias), "split K with bias, N=1001")


def test_gemm_ws_small_or_missing_workspace_is_gemm():
    M, N, K = 257, 2056, 4000
    x, w, ws = make_case(8, M, N, K)
    xq, xs = oracle.quant_act(x)
    args = (to_dev(xq), to_dev(xs), to_dev(w), to_dev(ws))
    ref = bf16_bits(bi8.gemm(*args))
    small = torch.empty((ws_bytes(M, N, K) - 16,), dtype=torch.uint8, device=device())
    assert np.array_equal(bf16_bits(bi8.gemm_ws(*args, small)), ref)
    assert np.array_equal(bf16_bits(bi8.gemm_ws(*args, None)), ref)
    # shapes that do not split ignore the workspace
    assert ws_bytes(4096, 4096, 4096) == 0 and ws_bytes(8, 4096, 4096) == 0 and ws_bytes(333, 5000, 4000) == 0
