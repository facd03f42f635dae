#!/usr/bin/env python3
"""Benchmark of the block-wise INT8 W8A8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input already
resident in HBM.  The default workload is the block-INT8 FusedMoE layer, the
largest of the measured configurations (4096 tokens, hidden 4096,
intermediate 14336, top-2 of 8 experts, [128,128] blocks): route, gather +
quantise, w13 grouped GEMM with the SiLU gating and requantisation as its
epilogue (two launches when a kernel variant is forced), w2 grouped GEMM,
combine.  The dense workloads (``--workload decode|prefill|...``) step
through dynamic activation quantisation (bf16 -> int8 + fp32 scales)
followed by the block-scaled int8 GEMM.

Weights rotate over enough distinct copies (>= 540 MB in total) that the
256 MB Infinity Cache cannot hold them, so HBM is what is measured.  K steps
are captured in one HIP graph and replayed once inside the timed region,
bracketed by synchronisation.

Prints ONE JSON line (rank 0, N=1) with the throughput, a ``roofline`` object
for the dominant kernel (its average launch time measured with HIP events on
its stream, and the average GFX clock over that timed region read from the
shader-clock counters), the same for the decode and prefill GEMMs under
``roofline_other`` (with the MoE default), and a ``cpu_baseline`` object (the
CPU oracle timed on a bounded sample of the same workload on this host, on
one core and on all the cores this process may use).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_wise_int8_amd as bi8  # noqa: E402
import workloads as wl  # noqa: E402

METRIC = "block-int8 GEMM TOPS + fraction of int8 MFMA/HBM roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
VARIANTS = {"auto": None, "skinny": bi8.GEMM_SKINNY, "128x64": bi8.GEMM_TILE_128X64,
            "256x128": bi8.GEMM_TILE_256X128, "256x256": bi8.GEMM_TILE_256X256}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items() if v is not None}
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POP/s)
PEAK_CLOCK_MHZ = 2400.0        # the GFX clock the published int8 peak assumes (256 CUs)
ROTATE_BYTES = 540 << 20       # > Infinity Cache (256 MB)
MAX_COPIES = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gemm_bytes(M, N, K, block=(128, 128)):
    """Algorithmic HBM bytes of one GEMM launch: xq + xs + w + ws + y."""
    NB, KB = bi8.scale_shape(N, K, *block)
    return M * K + 4 * M * KB + N * K + 4 * NB * KB + 2 * M * N


def quant_bytes(M, K):
    return 2 * M * K + M * K + 4 * M * bi8.scale_shape(1, K)[1]


def n_copies(weight_bytes, override=None):
    if override:
        return int(override)
    return int(max(1, min(MAX_COPIES, -(-ROTATE_BYTES // max(weight_bytes, 1)))))


class Dense:
    """quant_act + gemm on one [M, K] x [N, K] linear."""

    def __init__(self, name, copies=None, variant=None, per_channel=False):
        c = wl.CONFIGS[name]
        self.name = name
        self.variant = variant
        self.per_channel = per_channel
        self.M, self.N, self.K = c["M"], c["N"], c["K"]
        rng = wl.rng_for(c["seed"])
        self.x_np = wl.activations(rng, self.M, self.K, c.get("outlier_frac", 0.0))
        self.w_np = wl.weights(rng, self.N, self.K)
        # per-channel: blocks of 1 x K (one scale per weight row and per token)
        self.block = (1, self.K) if per_channel else (128, 128)
        self.ws_np = wl.weight_scales(rng, *bi8.scale_shape(self.N, self.K, *self.block))
        self.x = bf16_dev(self.x_np)
        w, ws = dev(self.w_np), dev(self.ws_np)
        self.copies = n_copies(self.N * self.K, copies)
        self.w = [w] + [w.clone() for _ in range(self.copies - 1)]
        self.ws = [ws] + [ws.clone() for _ in range(self.copies - 1)]
        KB = bi8.scale_shape(self.N, self.K, *self.block)[1]
        self.xq = torch.empty((self.M, self.K), dtype=torch.int8, device="cuda")
        self.xs = torch.empty((self.M, KB), dtype=torch.float32, device="cuda")
        self.y = torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")
        # the GEMM's caller workspace (split K on grids of few tiles), allocated once
        nws = 0 if per_channel or variant is not None else bi8.gemm_workspace_size(self.M, self.N, self.K)
        self.workspace = torch.empty((nws,), dtype=torch.uint8, device="cuda") if nws else None
        self.ops = 2 * self.M * self.N * self.K
        self.quant_shape = (self.M, self.K)
        self.dominant = "gemm_per_channel" if per_channel else "gemm"
        self.dominant_bytes = gemm_bytes(self.M, self.N, self.K, self.block)
        self.dominant_ops = self.ops
        outl = c.get("outlier_frac", 0.0)
        self.workload = ("%s linear M=%d K=%d N=%d %s%s" %
                         (name, self.M, self.K, self.N,
                          "per-channel (blocks 1 x K)" if per_channel else "block [128,128]",
                          ", %g%% outlier channels x%g" % (100 * outl, c["outlier_scale"]) if outl else ""))

    def quant(self, i):
        bi8.quant_act(self.x, self.xq, self.xs, block_k=self.block[1])

    def dominant_launch(self, i):
        j = i % self.copies
        if self.workspace is not None:
            bi8.gemm_ws(self.xq, self.xs, self.w[j], self.ws[j], self.workspace, y=self.y)
        else:
            bi8.gemm(self.xq, self.xs, self.w[j], self.ws[j], y=self.y, block=self.block, variant=self.variant)

    def step(self, i):
        self.quant(i)
        self.dominant_launch(i)

    def config(self):
        v = bi8.gemm_select(self.M, self.N, self.K) if self.variant is None else self.variant
        ws_bytes = 0 if self.workspace is None else self.workspace.numel()
        return {"workload": self.workload, "M": self.M, "K": self.K, "N": self.N,
                "block": list(self.block), "weight_copies": self.copies,
                "kernel": "per-channel" if self.per_channel else VARIANT_NAMES[v],
                "split_k": ws_bytes // (4 * self.M * self.N) if ws_bytes else 1}

    def cpu_sample(self, budget_s, threads=1):
        """Time the oracle (quant + GEMM) on a bounded sample of token rows.
        With threads > 1 the unchanged single-threaded oracle GEMM runs on
        disjoint slices of the weight rows (whole scale blocks), one per
        thread (the oracle's C code runs with the GIL released)."""
        import oracle
        bn = self.block[0]
        nblk = -(-self.N // bn)
        n_sl = max(1, min(threads, nblk))
        edges = [min(self.N, bn * (nblk * i // n_sl)) for i in range(n_sl + 1)]
        slices = [(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]
        oracle.scale_shape(1, 1)   # load the library before any thread does

        def gemm_slice(args):
            xq, xs, (a, b) = args
            return oracle.gemm(xq, xs, self.w_np[a:b], self.ws_np[a // bn:-(-b // bn)], block=self.block)

        with ThreadPoolExecutor(len(slices)) as ex:
            def once(rows):
                xq, xs = oracle.quant_act(self.x_np[:rows], block_k=self.block[1])
                list(ex.map(gemm_slice, [(xq, xs, sl) for sl in slices]))

            t0 = time.perf_counter()
            once(1)   # one row costs N*K MACs: size the sample from it
            t_row = max(time.perf_counter() - t0, 1e-4)
            rows = int(max(1, min(self.M, budget_s / t_row)))
            reps = int(max(1, min(1000, budget_s / (t_row * rows))))
            t0 = time.perf_counter()
            for _ in range(reps):
                once(rows)
            dt = time.perf_counter() - t0
        ops = 2.0 * rows * self.N * self.K * reps
        return ops / dt / 1e12, len(slices), (
            "%d of %d token rows x all N, quant+GEMM, %d repetition(s), %.1f s%s" %
            (rows, self.M, reps, dt, ", N split over %d threads" % len(slices) if len(slices) > 1 else ""))


class Moe:
    """The FusedMoE layer on the GPU, one launch per step: route (top-k of the
    softmax of the router logits, dispatch order), gather + quantise, w13
    grouped GEMM with SiLU gating + requantise in its epilogue (the two as
    separate launches when a kernel variant is forced), w2 grouped GEMM,
    weighted combine."""

    def __init__(self, variant=None):
        c = wl.CONFIGS["moe"]
        self.name = "moe"
        self.variant = variant
        T, H, I, E, k = c["T"], c["H"], c["I"], c["E"], c["topk"]
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        rng = wl.rng_for(c["seed"])
        self.x_np = wl.activations(rng, T, H)
        self.logits_np = wl.router_logits(rng, T, E)
        self.w13_np = wl.weights(rng, E, 2 * I, H)
        self.ws13_np = wl.weight_scales(rng, E, *bi8.scale_shape(2 * I, H))
        self.w2_np = wl.weights(rng, E, H, I)
        self.ws2_np = wl.weight_scales(rng, E, *bi8.scale_shape(H, I))
        self.R = T * k
        self.x = bf16_dev(self.x_np)
        self.logits = dev(self.logits_np)
        self.w13, self.ws13 = dev(self.w13_np), dev(self.ws13_np)
        self.w2, self.ws2 = dev(self.w2_np), dev(self.ws2_np)
        KB1, KB2 = bi8.scale_shape(1, H)[1], bi8.scale_shape(1, I)[1]
        d = dict(device="cuda")
        self.ids = torch.empty((T, k), dtype=torch.int32, **d)
        self.wts = torch.empty((T, k), dtype=torch.float32, **d)
        self.st = torch.empty((self.R,), dtype=torch.int32, **d)
        self.off = torch.empty((E + 1,), dtype=torch.int32, **d)
        self.row_of = torch.empty((T, k), dtype=torch.int32, **d)
        self.xq1 = torch.empty((self.R, H), dtype=torch.int8, **d)
        self.xs1 = torch.empty((self.R, KB1), dtype=torch.float32, **d)
        self.y13 = torch.empty((self.R, 2 * I), dtype=torch.bfloat16, **d)
        self.xq2 = torch.empty((self.R, I), dtype=torch.int8, **d)
        self.xs2 = torch.empty((self.R, KB2), dtype=torch.float32, **d)
        self.y2 = torch.empty((self.R, H), dtype=torch.bfloat16, **d)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, **d)
        # w2's workspace (the tiles of a partial last round split over K), as
        # the layer allocates it
        nb = bi8.moe_gemm_workspace_size(self.R, H, I, E) if variant is None else 0
        self.wsp2 = torch.empty(nb, dtype=torch.uint8, **d) if nb else None
        self.copies = 1
        self.quant_shape = (self.R, H)   # the gathered rows
        self.ops = 2 * self.R * (2 * I) * H + 2 * self.R * H * I
        self.fused = variant is None and I % 128 == 0
        self.dominant = "moe_gemm_w13_silu_quant" if self.fused else "moe_gemm_w13"
        self.dominant_ops = 2 * self.R * (2 * I) * H
        w13_in = self.R * H + 4 * self.R * KB1 + E * 2 * I * H + 4 * E * bi8.scale_shape(2 * I, H)[0] * KB1
        self.w13_bytes = w13_in + 2 * self.R * 2 * I
        self.fused_bytes = w13_in + self.R * I + 4 * self.R * KB2
        self.dominant_bytes = self.fused_bytes if self.fused else self.w13_bytes
        self.workload = ("moe layer T=%d tokens top-%d of E=%d, hidden %d, intermediate %d, "
                         "block [128,128]" % (T, k, E, H, I))
        self.route(0)
        self.quant(0)   # operands for the dominant kernel timed alone

    def route(self, i):
        bi8.moe_route(self.logits, self.k, out=(self.ids, self.wts, self.st, self.off, self.row_of))

    def quant(self, i):
        bi8.quant_act_gather(self.x, self.st, self.xq1, self.xs1)

    def launch_w2(self, i):
        bi8.moe_gemm(self.xq2, self.xs2, self.off, self.w2, self.ws2, y=self.y2, variant=self.variant,
                     workspace=self.wsp2)

    def launch_w13(self, i):
        bi8.moe_gemm(self.xq1, self.xs1, self.off, self.w13, self.ws13, y=self.y13, variant=self.variant)

    def launch_w13_gated(self, i):
        bi8.moe_gemm_silu_quant(self.xq1, self.xs1, self.off, self.w13, self.ws13, self.xq2, self.xs2)

    def dominant_launch(self, i):
        if self.fused:
            self.launch_w13_gated(i)
        else:
            self.launch_w13(i)

    def step(self, i):
        self.route(i)
        self.quant(i)
        if self.fused:
            self.launch_w13_gated(i)
        else:
            self.launch_w13(i)
            bi8.silu_mul_quant(self.y13, self.xq2, self.xs2)
        self.launch_w2(i)
        bi8.moe_combine(self.y2, self.row_of, self.wts, out=self.out)

    def parts(self):
        """Each step of the layer on its own: name -> (launch, algorithmic bytes)."""
        R, H, I, T, k = self.R, self.H, self.I, self.T, self.k
        KB1, KB2 = bi8.scale_shape(1, H)[1], bi8.scale_shape(1, I)[1]
        return {
            "route": (self.route, 4 * T * self.E + 4 * T * k * 4 + 4 * (self.E + 1)),
            "gather_quant": (self.quant, quant_bytes(R, H)),
            "moe_gemm_w13_silu_quant": (self.launch_w13_gated, self.fused_bytes),
            "moe_gemm_w13": (self.launch_w13, self.w13_bytes),
            "silu_mul_quant": (lambda i: bi8.silu_mul_quant(self.y13, self.xq2, self.xs2),
                               2 * R * 2 * I + R * I + 4 * R * KB2),
            "moe_gemm_w2": (self.launch_w2, R * I + 4 * R * KB2 + self.E * H * I + 2 * R * H),
            "combine": (lambda i: bi8.moe_combine(self.y2, self.row_of, self.wts, out=self.out),
                        2 * R * H + 8 * T * k + 2 * T * H),
        }

    def config(self):
        v = (bi8.moe_gemm_select(self.R, 2 * self.I, self.H, self.E) if self.variant is None
             else self.variant)
        v2 = (bi8.moe_gemm_select(self.R, self.H, self.I, self.E) if self.variant is None
              else self.variant)
        return {"workload": self.workload, "T": self.T, "E": self.E, "topk": self.k,
                "hidden": self.H, "intermediate": self.I, "rows": self.R, "block": [128, 128],
                "kernel": VARIANT_NAMES[v], "kernel_w2": VARIANT_NAMES[v2],
                "w13_gating_epilogue": self.fused}

    def cpu_sample(self, budget_s, threads=1):
        """Time the oracle's layer (route, quantise, w13 GEMM, SiLU, requantise,
        w2 GEMM, combine) on a bounded sample of tokens.  With threads > 1 the
        unchanged single-threaded oracle runs the layer on disjoint token
        slices, one per thread (each token's result depends on its own row
        only; the oracle's C code runs with the GIL released)."""
        import oracle
        ids, wts = oracle.topk_softmax(self.logits_np, self.k)

        def layer(tokens):
            st, off, row_of = oracle.moe_align(ids[tokens], self.E)
            xq, xs = oracle.quant_act(self.x_np[tokens][st])
            h = oracle.moe_gemm(xq, xs, off, self.w13_np, self.ws13_np)
            aq, as_ = oracle.quant_act(oracle.silu_mul(h))
            y2 = oracle.moe_gemm(aq, as_, off, self.w2_np, self.ws2_np)
            oracle.combine(y2, row_of, wts[tokens].astype(np.float32))
            return len(tokens)

        threads = max(1, min(threads, self.T))
        with ThreadPoolExecutor(threads) as ex:
            def run(n):
                edges = np.linspace(0, n, threads + 1).astype(int)
                return sum(ex.map(layer, [np.arange(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]))

            t0 = time.perf_counter()
            run(threads)   # one token per thread: size the sample from it
            t_round = max(time.perf_counter() - t0, 1e-4)
            n = int(max(threads, min(self.T, threads * budget_s / t_round)))
            t0 = time.perf_counter()
            done = run(n)
            dt = time.perf_counter() - t0
        ops = 2.0 * done * self.k * (2 * self.I * self.H + self.H * self.I)
        return ops / dt / 1e12, threads, (
            "first %d of %d tokens through the whole layer, %.1f s%s" %
            (done, self.T, dt, ", token slices over %d threads" % threads if threads > 1 else ""))


def make_workload(name, copies=None, variant=None, per_channel=False):
    if name == "moe":
        return Moe(variant)
    return Dense(name, copies, variant, per_channel)


def capture(fn, steps):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    return g


class ClockProbe:
    """Average GFX clock over a timed region, from the shader-clock counters.

    ``libbi8clock.so`` launches one-wave workgroups that record the
    shader-clock cycle counter, the constant-rate real-time counter and the
    compute unit they ran on.  One launch before and one after the region, on
    the same stream, give per compute unit: cycles / real time = the average
    clock there over the region (the launches bracket it, so the figure
    includes the few microseconds of launch gaps at its ends).  The cycle
    counters of different compute units do not agree with each other, so
    only samples of the same unit are compared; the XCD's figure is the
    median over its units."""

    BLOCKS = 1024   # about four per compute unit: every unit is sampled

    def __init__(self):
        path = os.path.join(ROOT, "block_wise_int8_amd", "libbi8clock.so")
        self.lib = ctypes.CDLL(path)
        self.lib.bi8clock_sample.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        self.lib.bi8clock_sample.restype = ctypes.c_int
        self.lib.bi8clock_wall_rate_khz.argtypes = [ctypes.c_int]
        self.lib.bi8clock_wall_rate_khz.restype = ctypes.c_int
        self.rate_khz = self.lib.bi8clock_wall_rate_khz(torch.cuda.current_device())
        self.buf = torch.zeros((2, self.BLOCKS, 3), dtype=torch.int64, device="cuda")

    def mark(self, i, stream):
        rc = self.lib.bi8clock_sample(ctypes.c_void_p(self.buf[i].data_ptr()), self.BLOCKS,
                                      ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("clock probe launch failed (%d)" % rc)

    @staticmethod
    def _units(sample):
        """{(xcd, CU / shader array / engine bits of HW_ID): (cycles, real time)}, first sample of each."""
        out = {}
        for t, r, place in sample.tolist():
            key = (place & 0xF, (place >> 40) & 0xFF)
            out.setdefault(key, (t, r))
        return out

    def read(self):
        """{"mhz": mean over XCDs, "min", "max" over XCDs, "xcds", "cus"} after both marks, or None."""
        if self.rate_khz <= 0:
            return None
        b = self.buf.cpu().numpy()
        u0, u1 = self._units(b[0]), self._units(b[1])
        per_xcd = {}
        for key in sorted(set(u0) & set(u1)):
            dt, dr = u1[key][0] - u0[key][0], u1[key][1] - u0[key][1]
            if dt > 0 and dr > 0:
                per_xcd.setdefault(key[0], []).append(dt / dr * self.rate_khz / 1e3)
        if not per_xcd:
            return None
        f = np.array([np.median(v) for v in per_xcd.values()])
        if not (100.0 <= f.mean() <= 4000.0):   # not a shader clock: do not report it
            return None
        return {"mhz": round(float(f.mean()), 1), "min": round(float(f.min()), 1),
                "max": round(float(f.max()), 1), "xcds": len(f),
                "cus": int(sum(len(v) for v in per_xcd.values()))}


SETTLE_S = 0.05   # default untimed GPU work before each timed region (see timed)


def timed(fn, steps, use_graph, clock=None, warmup=0):
    """Run ``steps`` calls of fn; return (wall seconds, event seconds, clock).

    Before the timed region the captured steps are replayed, untimed, for at
    least SETTLE_S seconds, then ``warmup`` untimed calls run right before
    it.  The GPU idles while a graph is captured and its clock drops; it takes
    some tens of milliseconds of back-to-back work to settle again (measured
    at 4096^3: 93-94 us per GEMM with no untimed launches before the region,
    88-89 us after 20, 84 us after 200 or more), so without the settling the
    timed region would measure the clock's ramp, not the kernels."""
    g = capture(fn, steps) if use_graph else None
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        if g is not None:
            g.replay()
        else:
            for i in range(steps):
                fn(i)
        torch.cuda.synchronize()
    if warmup:
        if use_graph:   # back to back on the GPU, as the timed steps run
            capture(fn, warmup).replay()
        else:
            for i in range(warmup):
                fn(i)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if clock is not None:
        clock.mark(0, stream)
    e0.record(stream)
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            fn(i)
    e1.record(stream)
    if clock is not None:
        clock.mark(1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1e3, (clock.read() if clock is not None else None)


def roofline(w, t_dom, clk):
    """The dominant kernel's roofline object: achieved / published peak, and
    the int8 peak scaled to the clock observed while it ran."""
    hbm_bound = w.dominant_ops / (INT8_PEAK_TOPS * 1e12) < w.dominant_bytes / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        achieved = w.dominant_bytes / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = w.dominant_ops / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
    roof["kernel"] = w.dominant
    roof["avg_launch_us"] = round(t_dom * 1e6, 3)
    roof["algorithmic_bytes"] = w.dominant_bytes
    roof["algorithmic_ops"] = w.dominant_ops
    roof["clock_mhz"] = clk
    if clk is not None and not hbm_bound:
        peak_clk = INT8_PEAK_TOPS * clk["mhz"] / PEAK_CLOCK_MHZ
        roof["peak_at_clock"] = round(peak_clk, 1)
        roof["frac_at_clock"] = round(achieved / peak_clk, 4)
    return roof


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_wise_int8_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs, or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="moe", choices=sorted(wl.CONFIGS))
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3,
                    help="untimed replays before each timed region, in ms of wall time (default %(default)g; "
                         "0 for profiler runs that count every dispatch)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for each cpu_baseline leg (one core, all cores)")
    ap.add_argument("--other", default="decode,prefill",
                    help="with the moe workload, also time the dominant GEMM of these dense workloads "
                         "(comma-separated; empty or 'none' for none) under roofline_other")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--variant", default="auto", choices=sorted(VARIANTS),
                    help="GEMM kernel (default: the library's shape-based choice)")
    ap.add_argument("--per-channel", action="store_true",
                    help="dense workloads in the per-channel form (blocks of 1 x K)")
    ap.add_argument("--copies", type=int, default=None,
                    help="weight copies to rotate over (default: enough to exceed the Infinity Cache)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (x16 launches), for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes, and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.randint(0, 127, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(16):
            torch.add(src, 1, out=dst)   # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 16}), flush=True)
        return

    SETTLE_S = max(0.0, args.settle_ms / 1e3)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the block-wise INT8 linear runs on one GPU's share "
              "here and no multi-GPU path is built (got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)

    bi8.load()
    log("[bench] setting up workload %s" % args.workload)
    if args.per_channel and args.workload == "moe":
        print("--per-channel applies to the dense workloads", file=sys.stderr)
        sys.exit(2)
    w = make_workload(args.workload, args.copies, VARIANTS[args.variant], args.per_channel)
    use_graph = not args.eager
    clock = ClockProbe()

    # the W warmup steps run right before the timed steps (after the graph
    # capture, which leaves the GPU idle, and after SETTLE_S of untimed
    # replays that let the GFX clock settle); every other timed region below
    # gets the same untimed work of its own right before it
    log("[bench] timing %d steps (%s) after %d warmup steps" %
        (args.steps, "graph" if use_graph else "eager", args.warmup))
    wall, ev, clk_step = timed(w.step, args.steps, use_graph, clock, warmup=args.warmup)
    ms_per_step = wall / args.steps * 1e3

    log("[bench] timing the dominant kernel (%s) alone" % w.dominant)
    _, ev_dom, clk_dom = timed(w.dominant_launch, args.steps, use_graph, clock, warmup=args.warmup)
    t_dom = ev_dom / args.steps
    _, ev_q, _ = timed(w.quant, args.steps, use_graph, warmup=args.warmup)
    t_q = ev_q / args.steps

    parts = None
    if hasattr(w, "parts"):
        parts = {}
        for name, (fn, nbytes) in w.parts().items():
            _, ev_p, _ = timed(fn, args.steps, use_graph, warmup=args.warmup)
            t_p = ev_p / args.steps
            parts[name] = {"avg_launch_us": round(t_p * 1e6, 3), "GB/s": round(nbytes / t_p / 1e9, 1)}
    value = w.ops / (wall / args.steps) / 1e12
    roof = roofline(w, t_dom, clk_dom)
    # the counters were taken with the default kernel choice of the block form
    roof["traffic"] = (counter_traffic(args.workload)
                       if args.variant == "auto" and not args.per_channel else None)

    others = None
    other_names = [n for n in args.other.split(",") if n and n != "none"]
    if args.workload == "moe" and other_names:
        others = {}
        for name in other_names:
            log("[bench] timing the dominant kernel of %s alone" % name)
            o = make_workload(name)
            o.quant(0)
            _, ev_o, clk_o = timed(o.dominant_launch, args.steps, use_graph, clock, warmup=args.warmup)
            r = roofline(o, ev_o / args.steps, clk_o)
            r["traffic"] = counter_traffic(name)
            r["config"] = o.config()
            others[name] = r
            del o
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": round(SETTLE_S * 1e3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic", "config": w.config(), "roofline": roof,
        "roofline_other": others,
        "clock_mhz_step": clk_step,
        "quant_act": {"avg_launch_us": round(t_q * 1e6, 3),
                      "GB/s": round(quant_bytes(*w.quant_shape) / t_q / 1e9, 1)},
        "steps_alone": parts,
        "event_ms_per_step": round(ev / args.steps * 1e3, 5),
        "timing": "hip graph of %d steps, one replay" % args.steps if use_graph else "eager launches",
    }
    if not args.no_cpu:
        cores = max(1, min(16, len(os.sched_getaffinity(0))))
        log("[bench] cpu baseline (oracle, one core, ~%.0f s)" % args.cpu_budget)
        v1, _, s1 = w.cpu_sample(args.cpu_budget, 1)
        log("[bench] cpu baseline (oracle, %d threads, ~%.0f s)" % (cores, args.cpu_budget))
        vn, used, sn = w.cpu_sample(args.cpu_budget, cores)
        out["cpu_baseline"] = {"value": round(vn, 6), "unit": "TOPS", "cores": used, "kind": "oracle",
                               "sample": sn, "cpu_model": cpu_model(),
                               "one_core": {"value": round(v1, 6), "cores": 1, "sample": s1}}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
