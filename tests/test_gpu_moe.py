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
from gpu_util import (GEMM_REL_TOL, assert_gemm_close, bf16_bits, bf16_to_dev, bits_to_f64, device, gemm_report, ordered,
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


FUSED_CASES = [
    # R, K, I, per-expert row counts (empty experts, ragged tails, several 256-row tiles)
    (700, 384, 256, [0, 300, 1, 399]),
    (513, 4096, 1408, [256, 0, 257]),
    (64, 128, 128, [64]),
    (1000, 400, 384, [10, 600, 0, 0, 390]),
    (1, 16, 128, [0, 1, 0]),            # one row, K of one partial block
    (300, 144, 256, [300]),             # one expert, a ragged second K block
    (129, 2048, 128, [128, 1]),         # a 128-row tile and a 1-row tile
]


@pytest.mark.parametrize("R,K,I,sizes", FUSED_CASES)
def test_moe_gemm_silu_quant_is_the_unfused_pipeline(R, K, I, sizes):
    """The w13 GEMM with the gating epilogue against the two launches it
    replaces (bit for bit), and that chain against the oracle: h within the
    GEMM tolerance, a within one bf16 ulp, codes and scales exactly on the
    GPU's own a.  One expert's gate block gets a large scale (SiLU's far
    negative branch and large products) and another's last 128 gate and up
    rows are zero (all-zero groups, scale 0)."""
    E = len(sizes)
    assert sum(sizes) == R
    rng = np.random.default_rng(R + K + I)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    x = wl.activations(rng, R, K)
    xq, xs = bi8.quant_act(bf16_to_dev(x))
    w13 = wl.weights(rng, E, 2 * I, K)
    ws13 = wl.weight_scales(rng, E, *oracle.scale_shape(2 * I, K))
    ws13[E - 1, 0, :] *= 4096.0                # gate rows 0..127 of the last expert
    w13[0, I - 128:I] = 0                      # expert 0: last gate group zero
    w13[0, 2 * I - 128:] = 0                   # and its up rows
    d_off, d_w, d_ws = to_dev(off), to_dev(w13), to_dev(ws13)

    h = bi8.moe_gemm(xq, xs, d_off, d_w, d_ws)
    for v in (bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256):
        assert torch.equal(bi8.moe_gemm(xq, xs, d_off, d_w, d_ws, variant=v).view(torch.int16),
                           h.view(torch.int16)), "variant %d" % v
    aq_u, as_u, a_u = bi8.silu_mul_quant(h, return_a=True)

    # outputs inside a larger allocation: the rows past R must stay untouched
    aq_buf = torch.full((R + 1, I), 0x5A, dtype=torch.int8, device=device())
    as_buf = torch.full((R + 1, I // 128), -7.0, dtype=torch.float32, device=device())
    aq, as_ = bi8.moe_gemm_silu_quant(xq, xs, d_off, d_w, d_ws, aq=aq_buf[:R], as_=as_buf[:R])
    torch.cuda.synchronize()
    assert torch.equal(aq, aq_u), "codes differ from moe_gemm + silu_mul_quant"
    assert torch.equal(as_.view(torch.int32), as_u.view(torch.int32)), "scales differ"
    assert torch.all(aq_buf[R] == 0x5A) and torch.all(as_buf[R] == -7.0)
    aq2, as2 = bi8.moe_gemm_silu_quant(xq, xs, d_off, d_w, d_ws)   # fresh outputs, same result
    assert torch.equal(aq2, aq) and torch.equal(as2, as_)

    hb, ab = bf16_bits(h), bf16_bits(a_u)
    xq_h, xs_h = xq.cpu().numpy(), xs.cpu().numpy()
    for e in range(E):
        a0, b0 = int(off[e]), int(off[e + 1])
        if a0 == b0:
            continue
        rows = np.unique(np.concatenate([[a0, b0 - 1], rng.integers(a0, b0, 6)]))
        ref = oracle.gemm(xq_h[rows], xs_h[rows], w13[e], ws13[e])
        assert_gemm_close(hb[rows], ref, "h expert %d" % e)
    assert_bf16_near(ab, oracle.silu_mul(hb), "silu*up", exact_frac=0.995)
    q_ref, s_ref = oracle.quant_act(ab)
    assert np.array_equal(aq.cpu().numpy(), q_ref) and np.array_equal(as_.cpu().numpy(), s_ref)
    z = as_.cpu().numpy()
    if sizes[0]:
        assert np.all(z[:sizes[0], -1] == 0.0)   # the zeroed group
    assert np.all(np.isfinite(z)) and np.all(z[:, :] >= 0)


WS_CASES = [
    # R, N, K, per-expert rows: every tile split (32 tiles, K in 3 blocks); 512
    # full tiles and a split tail of 32; 256 tiles exactly (no tail, no split);
    # a tail of 1 tile
    (700, 1024, 384, [0, 300, 1, 399]),
    (4100, 4096, 2048, [1025, 1000, 1075, 1000]),
    (2048, 4096, 1024, [1024, 1024]),
    (2049, 4096, 512, [1024, 1025]),
    # one expert of 33 m-tiles (three tile groups), tail tiles split
    (4300, 2048, 512, [4200, 100]),
]


@pytest.mark.parametrize("R,N,K,sizes", WS_CASES)
def test_moe_gemm_ws_split_tail(R, N, K, sizes):
    """The grouped GEMM with a workspace (the last, partial round's tiles split
    over K) against the one without (the tiles of the full rounds bit for bit,
    the split tiles within the fp32 reassociation of their sums: one bf16 ulp)
    and against the oracle on rows in every tile; with exactly representable
    sums the two forms agree bit for bit everywhere."""
    E = len(sizes)
    rng = np.random.default_rng(R + N + K)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    xq = rng.integers(-127, 128, (R, K), dtype=np.int8)
    xs = (rng.random((R, (K + 127) // 128)) * 1e-2 + 1e-3).astype(np.float32)
    w = wl.weights(rng, E, N, K)
    ws = wl.weight_scales(rng, E, *oracle.scale_shape(N, K))
    nbytes = bi8.moe_gemm_workspace_size(R, N, K, E)
    assert nbytes > 0, "the case must take the 256 x 128 kernel"
    wsp = torch.empty(nbytes, dtype=torch.uint8, device=device())
    d = [to_dev(a) for a in (xq, xs, off, w, ws)]
    plain = bf16_bits(bi8.moe_gemm(*d))
    y_buf = torch.full((R + 1, N), -1.0, dtype=torch.bfloat16, device=device())
    split = bf16_bits(bi8.moe_gemm(*d, y=y_buf[:R], workspace=wsp))
    assert np.all(bf16_bits(y_buf[R]) == bf16_bits(torch.tensor([-1.0], dtype=torch.bfloat16))[0])
    assert np.all(np.isfinite(bits_to_f64(split)))
    # reassociated fp32 sums: within a bf16 ulp of the row's largest output
    # (relative to a single output near zero the difference may be larger)
    g, r = bits_to_f64(split), bits_to_f64(plain)
    row_max = np.abs(r).max(axis=1, keepdims=True)
    assert np.all(np.abs(g - r) <= 2.0 ** -7 * row_max), "split tail outside the reassociation bound"
    assert np.mean(split == plain) >= 0.99
    split2 = bf16_bits(bi8.moe_gemm(*d, workspace=wsp))   # the workspace is reused: same result
    assert np.array_equal(split, split2)
    for e, rows in segment_tile_rows(off, 128, rng):
        ref = oracle.gemm(xq[rows], xs[rows], w[e], ws[e])
        assert_gemm_close(split[rows], ref, "expert %d" % e)
    # exact sums: codes in [-3, 3], power-of-two scales
    xq_e = rng.integers(-3, 4, (R, K), dtype=np.int8)
    w_e = rng.integers(-3, 4, (E, N, K), dtype=np.int8)
    xs_e = np.exp2(rng.integers(-4, 1, xs.shape)).astype(np.float32)
    ws_e = np.exp2(rng.integers(-4, 1, ws.shape)).astype(np.float32)
    d_e = [to_dev(a) for a in (xq_e, xs_e, off, w_e, ws_e)]
    assert np.array_equal(bf16_bits(bi8.moe_gemm(*d_e, workspace=wsp)), bf16_bits(bi8.moe_gemm(*d_e)))


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


# ------------------------------------------------ the full-size MoE layer --
#
# The MoE workload at its real size (4096 tokens, hidden 4096, intermediate
# 14336, top-2 of 8 experts), drawn exactly as the benchmark draws it, run
# step by step on the GPU with every intermediate kept.  Every stage is
# compared with the oracle on rows sampled in every 128-row tile of every
# expert segment (so in every tile of each grouped-GEMM kernel, whose tiles
# start at the segment starts), each fed the GPU's previous stage; and the
# layer end to end on 64 tokens covering every expert, against the oracle's
# pipeline computed from the inputs alone.

MOE_VARIANTS = [None, "ws", bi8.GEMM_TILE_256X128, bi8.GEMM_TILE_256X256]   # "ws": default with a workspace


@pytest.fixture(scope="module")
def moe_full():
    c = wl.CONFIGS["moe"]
    T, H, I, E, k = c["T"], c["H"], c["I"], c["E"], c["topk"]
    rng = wl.rng_for(c["seed"])
    x = wl.activations(rng, T, H)
    logits = wl.router_logits(rng, T, E)
    w13 = wl.weights(rng, E, 2 * I, H)
    ws13 = wl.weight_scales(rng, E, *oracle.scale_shape(2 * I, H))
    w2 = wl.weights(rng, E, H, I)
    ws2 = wl.weight_scales(rng, E, *oracle.scale_shape(H, I))
    d = dict(x=bf16_to_dev(x), logits=to_dev(logits), w13=to_dev(w13), ws13=to_dev(ws13), w2=to_dev(w2),
             ws2=to_dev(ws2))
    ids, wts, st, off, row_of = bi8.moe_route(d["logits"], k)
    xq1, xs1 = bi8.quant_act_gather(d["x"], st)
    h = bi8.moe_gemm(xq1, xs1, off, d["w13"], d["ws13"])
    aq, as_, a = bi8.silu_mul_quant(h, return_a=True)
    # w2 as the layer runs it: with a workspace for a split last round
    wsp_bytes = bi8.moe_gemm_workspace_size(aq.shape[0], H, I, E)
    wsp = torch.empty(wsp_bytes, dtype=torch.uint8, device=device()) if wsp_bytes else None
    y2 = bi8.moe_gemm(aq, as_, off, d["w2"], d["ws2"], workspace=wsp)
    out = bi8.moe_combine(y2, row_of, wts)
    out_layer = bi8.moe_layer(d["x"], d["logits"], d["w13"], d["ws13"], d["w2"], d["ws2"], k)
    aq_f, as_f = bi8.moe_gemm_silu_quant(xq1, xs1, off, d["w13"], d["ws13"])
    torch.cuda.synchronize()
    host = dict(T=T, H=H, I=I, E=E, k=k, x=x, logits=logits, w13=w13, ws13=ws13, w2=w2, ws2=ws2,
                ids=ids.cpu().numpy(), wts=wts.cpu().numpy(), st=st.cpu().numpy(), off=off.cpu().numpy(),
                row_of=row_of.cpu().numpy(), out=bf16_bits(out), out_layer=bf16_bits(out_layer))
    dev = dict(d, xq1=xq1, xs1=xs1, h=h, aq=aq, as_=as_, a=a, y2=y2, off=off, aq_f=aq_f, as_f=as_f, wsp=wsp)
    yield host, dev
    del dev, d
    torch.cuda.empty_cache()


def segment_tile_rows(off, bm, rng):
    """Per expert: rows drawn in every bm-row tile of its segment, plus its
    first and last row."""
    rows = []
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        r = {a, b - 1}
        for t0 in range(a, b, bm):
            r.add(int(rng.integers(t0, min(b, t0 + bm))))
        rows.append((e, np.array(sorted(r))))
    return rows


def oracle_rows_pooled(fn, items):
    """Apply a per-item oracle computation on a thread pool (each call of the
    unchanged single-threaded oracle works on its own rows)."""
    from concurrent.futures import ThreadPoolExecutor
    from gpu_util import host_threads
    oracle.scale_shape(1, 1)   # load the library once, before the threads
    with ThreadPoolExecutor(host_threads()) as ex:
        return list(ex.map(fn, items))


def test_moe_full_size_route(moe_full):
    host, _ = moe_full
    ids_r, w_r = oracle.topk_softmax(host["logits"], host["k"])
    st_r, off_r, row_of_r = oracle.moe_align(ids_r, host["E"])
    assert np.array_equal(host["ids"], ids_r)
    np.testing.assert_allclose(host["wts"], w_r, rtol=2e-6, atol=1e-30)
    assert np.array_equal(host["off"], off_r) and np.array_equal(host["st"], st_r)
    assert np.array_equal(host["row_of"], row_of_r)
    assert np.all(np.diff(off_r) > 0), "every expert receives rows"


@pytest.mark.parametrize("variant", MOE_VARIANTS)
def test_moe_full_size_grouped_gemms(moe_full, variant):
    """w13 on the gathered codes and w2 on the GPU's own SiLU-requantised
    activations, in each grouped-GEMM kernel, on rows in every tile."""
    host, dev = moe_full
    off = host["off"]
    samples = segment_tile_rows(off, 128, np.random.default_rng(11))
    xq1, xs1 = dev["xq1"].cpu().numpy(), dev["xs1"].cpu().numpy()
    aq, as_ = dev["aq"].cpu().numpy(), dev["as_"].cpu().numpy()
    for e, rows in samples:
        q_ref, s_ref = oracle.quant_act(host["x"][host["st"][rows]])
        assert np.array_equal(xq1[rows], q_ref) and np.array_equal(xs1[rows], s_ref)
    v = None if variant == "ws" else variant
    h = bf16_bits(bi8.moe_gemm(dev["xq1"], dev["xs1"], dev["off"], dev["w13"], dev["ws13"], variant=v))
    y2 = bf16_bits(bi8.moe_gemm(dev["aq"], dev["as_"], dev["off"], dev["w2"], dev["ws2"], variant=v,
                                workspace=dev["wsp"] if variant == "ws" else None))
    assert np.all(np.isfinite(bits_to_f64(h))) and np.all(np.isfinite(bits_to_f64(y2)))
    if variant in (None, "ws"):   # the layer's own w13 is the default kernel's
        assert np.array_equal(h, bf16_bits(dev["h"]))
    if variant == "ws":           # and its w2 runs with the workspace
        assert np.array_equal(y2, bf16_bits(dev["y2"]))
    refs = oracle_rows_pooled(
        lambda er: (oracle.gemm(xq1[er[1]], xs1[er[1]], host["w13"][er[0]], host["ws13"][er[0]]),
                    oracle.gemm(aq[er[1]], as_[er[1]], host["w2"][er[0]], host["ws2"][er[0]])), samples)
    for (e, rows), (r13, r2) in zip(samples, refs):
        assert_gemm_close(h[rows], r13, "w13 expert %d variant %s" % (e, variant))
        assert_gemm_close(y2[rows], r2, "w2 expert %d variant %s" % (e, variant))


def test_moe_full_size_silu_and_combine_stagewise(moe_full):
    host, dev = moe_full
    rows = np.concatenate([r for _, r in segment_tile_rows(host["off"], 128, np.random.default_rng(12))])
    h, a = bf16_bits(dev["h"][rows]), bf16_bits(dev["a"][rows])
    assert_bf16_near(a, oracle.silu_mul(h), "silu*up", exact_frac=0.995)
    q_ref, s_ref = oracle.quant_act(a)
    assert np.array_equal(dev["aq"][rows].cpu().numpy(), q_ref)
    assert np.array_equal(dev["as_"][rows].cpu().numpy(), s_ref)
    tokens = np.random.default_rng(13).choice(host["T"], 256, replace=False)
    y2 = bf16_bits(dev["y2"])
    ro = host["row_of"][tokens]
    wn = host["wts"][tokens]
    ref = oracle.combine(y2, ro, wn)
    out = host["out"][tokens]
    # the fp32 bound of the combine, as in test_combine_stagewise
    g, r = bits_to_f64(out), bits_to_f64(ref)
    mag = np.abs(wn[:, :, None].astype(np.float64) * bits_to_f64(y2)[ro]).sum(axis=1)
    ulp = np.abs(r) * 2.0 ** -7 + 2.0 ** -133
    assert np.all(np.abs(g - r) <= ulp + host["k"] * 2.0 ** -23 * mag), "combine outside the fp32 bound"
    assert np.mean(out == ref) >= 0.99


def test_moe_full_size_fused_gating_is_bit_identical(moe_full):
    """At the full layer size the fused w13 + gating launch writes exactly
    the codes and scales of the two launches it replaces (which the tests
    above hold to the oracle stage by stage)."""
    _, dev = moe_full
    assert torch.equal(dev["aq_f"], dev["aq"])
    assert torch.equal(dev["as_f"].view(torch.int32), dev["as_"].view(torch.int32))


def test_moe_full_size_layer_end_to_end(moe_full):
    """64 tokens, 8 routed to each expert, through the oracle's whole pipeline
    (route, quantise, w13, SiLU gating, requantise, w2, combine) from the
    inputs alone, against the GPU layer's output rows, within the stated
    tolerance over the sample and on every token row."""
    host, _ = moe_full
    k, E = host["k"], host["E"]
    ids_r, w_r = oracle.topk_softmax(host["logits"], k)
    rng = np.random.default_rng(14)
    tokens = []
    for e in range(E):
        cand = np.setdiff1d(np.nonzero(np.any(ids_r == e, axis=1))[0], tokens)
        tokens.extend(int(t) for t in rng.choice(cand, 8, replace=False))
    tokens = np.array(sorted(tokens))
    assert len(tokens) == 64 and set(ids_r[tokens].reshape(-1)) == set(range(E))

    def one_token(t):
        q, s = oracle.quant_act(host["x"][t:t + 1])
        rows = []
        for slot in range(k):
            e = int(ids_r[t, slot])
            hh = oracle.gemm(q, s, host["w13"][e], host["ws13"][e])
            aq, as_ = oracle.quant_act(oracle.silu_mul(hh))
            rows.append(oracle.gemm(aq, as_, host["w2"][e], host["ws2"][e])[0])
        return oracle.combine(np.stack(rows), np.arange(k, dtype=np.int32)[None, :],
                              w_r[t:t + 1].astype(np.float32))[0]

    ref = np.stack(oracle_rows_pooled(one_token, tokens))
    got = host["out"][tokens]
    assert np.all(np.isfinite(bits_to_f64(host["out"]))), "non-finite layer output"
    rel, frac_gt1, maxulp = gemm_report(got, ref)
    ulps = np.abs(ordered(got) - ordered(ref))
    hist = {u: float(np.mean(ulps == u)) for u in range(4)}
    what = "moe layer: max rel err %.3e, %.2f%% > 1 ulp, max %d ulp, share at 0..3 ulp %s" % (
        rel, 100 * frac_gt1, maxulp, hist)
    print(what)
    assert rel <= GEMM_REL_TOL, what
    # The stated tolerance per token row as well: a wrong expert, weight or
    # dropped slot for any token fails it.  (Bit-level agreement is not a
    # criterion end to end: where the binary64 and fp32 w13 sums round to
    # neighbouring bf16 values, SiLU and the requantised codes can move, and
    # each code step moves a w2 output by about 2e-4 of its size at
    # I = 14336, across a bf16 rounding boundary in a few percent of outputs;
    # the stage-wise tests above hold each stage to the one-ulp rules.)
    g, r = bits_to_f64(got), bits_to_f64(ref)
    per_tok = np.abs(g - r).max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-30)
    assert per_tok.max() <= GEMM_REL_TOL, "token %d: rel err %.3e" % (tokens[per_tok.argmax()], per_tok.max())
    # the one-call layer runs the same kernels: bit-identical
    assert np.array_equal(host["out_layer"], host["out"])
