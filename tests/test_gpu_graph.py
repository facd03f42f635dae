"""HIP-graph capture of the hot path: every replay equals the eager launch.

Steps are timed as HIP graphs, and callers that cannot allocate capture the
calls too.  The path enqueues no memset and no host synchronisation (the
grouped GEMM decodes its tiles from ``expert_offsets`` on the device, the
split tail's plan included), so a captured call must give, on every replay,
bit for bit what the same call gives eagerly on the inputs that the captured
buffers hold at that replay.  Each test replays the graph several times with
fresh inputs copied into the captured buffers, and runs the eager reference
(the same kernels on other buffers) and a synchronisation between replays.
Correctness against the oracle is the other GPU tests' business; here the
eager launch is the reference.
"""
import numpy as np
import pytest
import torch

import block_wise_int8_amd as bi8
import workloads as wl
from gpu_util import bf16_to_dev, device, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def dense_case(seed, M, N, K, bias=False):
    rng = wl.rng_for(seed)
    xs = [bf16_to_dev(wl.activations(rng, M, K, 0.01)) for _ in range(REPLAYS + 1)]
    NB, KB = bi8.scale_shape(N, K)
    w = to_dev(wl.weights(rng, N, K))
    ws = to_dev(wl.weight_scales(rng, NB, KB))
    b = bf16_to_dev(wl.activations(rng, 1, N)[0]) if bias else None
    return xs, w, ws, b


def replay_and_check(capture_fn, set_inputs, outputs, eager_fn):
    """Warm up, capture capture_fn, then for replay r = 1..REPLAYS: copy input
    set r into the captured buffers, replay, and compare every captured output
    with eager_fn(r)."""
    capture_fn()   # eager warm-up: loads the code objects outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_fn()
    for r in range(1, REPLAYS + 1):
        set_inputs(r)
        g.replay()
        torch.cuda.synchronize()
        ref = eager_fn(r)
        torch.cuda.synchronize()
        for name, out, want in zip(ref.keys(), outputs(), ref.values()):
            assert same_bits(out, want), "replay %d: %s differs from the eager launch" % (r, name)


@pytest.mark.parametrize("M,N,K,kernel,bias", [
    (8, 4096, 1024, bi8.GEMM_SKINNY, False),
    (333, 1000, 640, bi8.GEMM_TILE_128X64, True),
    (2048, 4096, 256, bi8.GEMM_TILE_256X128, False),
    (4096, 4096, 256, bi8.GEMM_TILE_256X256, True),
])
def test_linear_graph_replays_equal_eager(M, N, K, kernel, bias):
    assert bi8.gemm_select(M, N, K) == kernel
    xs_in, w, ws, b = dense_case((11, M, N, K), M, N, K, bias)
    dev = device()
    KB = bi8.scale_shape(N, K)[1]
    x = xs_in[0].clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty((M, KB), dtype=torch.float32, device=dev)

    def eager(r):
        q = torch.empty_like(xq)
        s = torch.empty_like(xsc)
        yy = bi8.linear(xs_in[r], w, ws, b, xq=q, xs=s)
        return {"y": yy, "xq": q, "xs": s}

    replay_and_check(lambda: bi8.linear(x, w, ws, b, y=y, xq=xq, xs=xsc),
                     lambda r: x.copy_(xs_in[r]), lambda: (y, xq, xsc), eager)


def test_split_k_gemm_graph_replays_equal_eager():
    M, N, K = 64, 8192, 4096
    nbytes = bi8.gemm_workspace_size(M, N, K)
    assert nbytes > 0, "the shape must take the split-K path"
    xs_in, w, ws, _ = dense_case((12, M, N, K), M, N, K)
    dev = device()
    qs = [bi8.quant_act(x) for x in xs_in]
    xq, xsc = qs[0][0].clone(), qs[0][1].clone()
    wsp = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def set_inputs(r):
        xq.copy_(qs[r][0])
        xsc.copy_(qs[r][1])

    def eager(r):
        other = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return {"y": bi8.gemm_ws(qs[r][0], qs[r][1], w, ws, other)}

    replay_and_check(lambda: bi8.gemm_ws(xq, xsc, w, ws, wsp, y=y), set_inputs, lambda: (y,), eager)


def test_linear_noalloc_graph_replays_equal_eager():
    M, N, K = 24, 4096, 2048
    xs_in, w, ws, b = dense_case((13, M, N, K), M, N, K, bias=True)
    x = xs_in[0].clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=device())
    replay_and_check(lambda: bi8.linear_noalloc(x, w, ws, b, y=y), lambda r: x.copy_(xs_in[r]), lambda: (y,),
                     lambda r: {"y": bi8.linear(xs_in[r], w, ws, b)})


def valid_w2_tiles(offsets: np.ndarray, H: int) -> int:
    rows = np.diff(offsets)
    return int(((rows + 127) // 128).sum()) * ((H + 255) // 256)


def test_moe_layer_graph_replays_equal_eager():
    """The whole layer with the routing changing from replay to replay: the
    expert segments, the grouped grids' valid tiles and the w2 split tail all
    follow the captured buffers' contents."""
    T, H, I, E, k = 1100, 4096, 256, 8, 2
    rng = wl.rng_for((14, T))
    xs_in = [bf16_to_dev(wl.activations(rng, T, H)) for _ in range(REPLAYS + 1)]
    logits_in = [to_dev(wl.router_logits(rng, T, E)) for _ in range(REPLAYS + 1)]
    w13 = to_dev(wl.weights(rng, E, 2 * I, H))
    ws13 = to_dev(wl.weight_scales(rng, E, *bi8.scale_shape(2 * I, H)))
    w2 = to_dev(wl.weights(rng, E, H, I))
    ws2 = to_dev(wl.weight_scales(rng, E, *bi8.scale_shape(H, I)))
    assert bi8.moe_gemm_workspace_size(T * k, H, I, E) > 0
    # every replay's routing leaves a partial last round of w2 tiles: the split tail runs
    for r in range(1, REPLAYS + 1):
        off = bi8.moe_route(logits_in[r], k)[3].cpu().numpy()
        tiles = valid_w2_tiles(off, H)
        assert tiles > 256 and tiles % 256 != 0, tiles

    x = xs_in[0].clone()
    logits = logits_in[0].clone()
    out = []

    def capture():
        out.clear()
        out.append(bi8.moe_layer(x, logits, w13, ws13, w2, ws2, k))

    def set_inputs(r):
        x.copy_(xs_in[r])
        logits.copy_(logits_in[r])

    replay_and_check(capture, set_inputs, lambda: (out[0],),
                     lambda r: {"out": bi8.moe_layer(xs_in[r], logits_in[r], w13, ws13, w2, ws2, k)})
