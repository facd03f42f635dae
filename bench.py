#!/usr/bin/env python3
"""Benchmark of the block-wise INT8 W8A8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input already
resident in HBM: dynamic activation quantisation (bf16 -> int8 + fp32 scales)
followed by the block-scaled int8 GEMM (the grouped GEMM for ``moe``: both
w13 and w2 projections, each with its quantisation pass).  The default
workload is the decode-shaped linear, M=8 tokens, K=N=4096, [128,128] blocks.

Weights rotate over enough distinct copies (>= 540 MB in total) that the
256 MB Infinity Cache cannot hold them, so HBM is what is measured.  K steps
are captured in one HIP graph and replayed once inside the timed region,
bracketed by synchronisation.

Prints ONE JSON line (rank 0, N=1) with the throughput, a ``roofline`` object
for the dominant kernel (its average launch time measured with HIP events on
its stream) and a ``cpu_baseline`` object (the CPU oracle timed on a bounded
sample of the same workload, on this host).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

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
        bi8.gemm(self.xq, self.xs, self.w[j], self.ws[j], y=self.y, block=self.block, variant=self.variant)

    def step(self, i):
        self.quant(i)
        self.dominant_launch(i)

    def config(self):
        v = bi8.gemm_select(self.M, self.N, self.K) if self.variant is None else self.variant
        return {"workload": self.workload, "M": self.M, "K": self.K, "N": self.N,
                "block": list(self.block), "weight_copies": self.copies,
                "kernel": "per-channel" if self.per_channel else VARIANT_NAMES[v]}

    def cpu_sample(self, budget_s):
        """Time the oracle (quant + GEMM) on a bounded sample of rows."""
        import oracle
        # one row costs N*K MACs; pick rows to fill roughly the budget
        t0 = time.perf_counter()
        xq, xs = oracle.quant_act(self.x_np[:1], block_k=self.block[1])
        oracle.gemm(xq, xs, self.w_np, self.ws_np, block=self.block)
        t_row = max(time.perf_counter() - t0, 1e-4)
        rows = int(max(1, min(self.M, budget_s / t_row)))
        reps = int(max(1, min(1000, budget_s / (t_row * rows))))
        t0 = time.perf_counter()
        for _ in range(reps):
            xq, xs = oracle.quant_act(self.x_np[:rows], block_k=self.block[1])
            oracle.gemm(xq, xs, self.w_np, self.ws_np, block=self.block)
        dt = time.perf_counter() - t0
        ops = 2.0 * rows * self.N * self.K * reps
        return ops / dt / 1e12, "%d of %d token rows x all N, quant+GEMM, %d repetition(s), %.1f s" % (
            rows, self.M, reps, dt)


class Moe:
    """The FusedMoE layer on the GPU, one launch per step: route (top-k of the
    softmax of the router logits, dispatch order), gather + quantise, w13
    grouped GEMM, SiLU gating + requantise, w2 grouped GEMM, weighted combine."""

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
        self.copies = 1
        self.quant_shape = (self.R, H)   # the gathered rows
        self.ops = 2 * self.R * (2 * I) * H + 2 * self.R * H * I
        self.dominant = "moe_gemm_w13"
        self.dominant_ops = 2 * self.R * (2 * I) * H
        self.dominant_bytes = (self.R * H + 4 * self.R * KB1 + E * 2 * I * H
                               + 4 * E * bi8.scale_shape(2 * I, H)[0] * KB1 + 2 * self.R * 2 * I)
        self.workload = ("moe layer T=%d tokens top-%d of E=%d, hidden %d, intermediate %d, "
                         "block [128,128]" % (T, k, E, H, I))
        self.route(0)
        self.quant(0)   # operands for the dominant kernel timed alone

    def route(self, i):
        bi8.moe_route(self.logits, self.k, out=(self.ids, self.wts, self.st, self.off, self.row_of))

    def quant(self, i):
        bi8.quant_act_gather(self.x, self.st, self.xq1, self.xs1)

    def dominant_launch(self, i):
        bi8.moe_gemm(self.xq1, self.xs1, self.off, self.w13, self.ws13, y=self.y13, variant=self.variant)

    def step(self, i):
        self.route(i)
        self.quant(i)
        self.dominant_launch(i)
        bi8.silu_mul_quant(self.y13, self.xq2, self.xs2)
        bi8.moe_gemm(self.xq2, self.xs2, self.off, self.w2, self.ws2, y=self.y2, variant=self.variant)
        bi8.moe_combine(self.y2, self.row_of, self.wts, out=self.out)

    def parts(self):
        """Each step of the layer on its own: name -> (launch, algorithmic bytes)."""
        R, H, I, T, k = self.R, self.H, self.I, self.T, self.k
        KB1, KB2 = bi8.scale_shape(1, H)[1], bi8.scale_shape(1, I)[1]
        return {
            "route": (self.route, 4 * T * self.E + 4 * T * k * 4 + 4 * (self.E + 1)),
            "gather_quant": (self.quant, quant_bytes(R, H)),
            "moe_gemm_w13": (self.dominant_launch, self.dominant_bytes),
            "silu_mul_quant": (lambda i: bi8.silu_mul_quant(self.y13, self.xq2, self.xs2),
                               2 * R * 2 * I + R * I + 4 * R * KB2),
            "moe_gemm_w2": (lambda i: bi8.moe_gemm(self.xq2, self.xs2, self.off, self.w2, self.ws2, y=self.y2,
                                                   variant=self.variant),
                            R * I + 4 * R * KB2 + self.E * H * I + 2 * R * H),
            "combine": (lambda i: bi8.moe_combine(self.y2, self.row_of, self.wts, out=self.out),
                        2 * R * H + 8 * T * k + 2 * T * H),
        }

    def config(self):
        v = (bi8.moe_gemm_select(self.R, 2 * self.I, self.H, self.E) if self.variant is None
             else self.variant)
        return {"workload": self.workload, "T": self.T, "E": self.E, "topk": self.k,
                "hidden": self.H, "intermediate": self.I, "rows": self.R, "block": [128, 128],
                "kernel": VARIANT_NAMES[v]}

    def cpu_sample(self, budget_s):
        """Time the oracle's layer (route, quantise, w13 GEMM, SiLU, requantise,
        w2 GEMM, combine) on a bounded sample of tokens."""
        import oracle
        ids, wts = oracle.topk_softmax(self.logits_np, self.k)

        def layer(tokens):
            n = len(tokens)
            st, off, row_of = oracle.moe_align(ids[tokens], self.E)
            xq, xs = oracle.quant_act(self.x_np[tokens][st])
            h = oracle.moe_gemm(xq, xs, off, self.w13_np, self.ws13_np)
            aq, as_ = oracle.quant_act(oracle.silu_mul(h))
            y2 = oracle.moe_gemm(aq, as_, off, self.w2_np, self.ws2_np)
            oracle.combine(y2, row_of, wts[tokens].astype(np.float32))
            return n

        t0 = time.perf_counter()
        layer(np.arange(1))
        t_tok = max(time.perf_counter() - t0, 1e-4)
        n = int(max(1, min(self.T, budget_s / t_tok)))
        t0 = time.perf_counter()
        layer(np.arange(n))
        dt = time.perf_counter() - t0
        ops = 2.0 * n * self.k * (2 * self.I * self.H + self.H * self.I)
        return ops / dt / 1e12, "first %d of %d tokens through the whole layer, %.1f s" % (n, self.T, dt)


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


def timed(fn, steps, use_graph):
    """Run ``steps`` calls of fn; return (wall seconds, event seconds)."""
    g = capture(fn, steps) if use_graph else None
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1e3


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
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(wl.CONFIGS))
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for cpu_baseline")
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

    log("[bench] warmup %d steps" % args.warmup)
    for i in range(args.warmup):
        w.step(i)
    torch.cuda.synchronize()

    log("[bench] timing %d steps (%s)" % (args.steps, "graph" if use_graph else "eager"))
    wall, ev = timed(w.step, args.steps, use_graph)
    ms_per_step = wall / args.steps * 1e3

    log("[bench] timing the dominant kernel (%s) alone" % w.dominant)
    _, ev_dom = timed(w.dominant_launch, args.steps, use_graph)
    t_dom = ev_dom / args.steps
    _, ev_q = timed(w.quant, args.steps, use_graph)
    t_q = ev_q / args.steps

    parts = None
    if hasattr(w, "parts"):
        parts = {}
        for name, (fn, nbytes) in w.parts().items():
            _, ev_p = timed(fn, args.steps, use_graph)
            t_p = ev_p / args.steps
            parts[name] = {"avg_launch_us": round(t_p * 1e6, 3), "GB/s": round(nbytes / t_p / 1e9, 1)}
    value = w.ops / (wall / args.steps) / 1e12
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
    # the counters were taken with the default kernel choice of the block form
    roof["traffic"] = (counter_traffic(args.workload)
                       if args.variant == "auto" and not args.per_channel else None)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic", "config": w.config(), "roofline": roof,
        "quant_act": {"avg_launch_us": round(t_q * 1e6, 3),
                      "GB/s": round(quant_bytes(*w.quant_shape) / t_q / 1e9, 1)},
        "steps_alone": parts,
        "event_ms_per_step": round(ev / args.steps * 1e3, 5),
        "timing": "hip graph of %d steps, one replay" % args.steps if use_graph else "eager launches",
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle, ~%.0f s)" % args.cpu_budget)
        cpu_tops, sample = w.cpu_sample(args.cpu_budget)
        out["cpu_baseline"] = {"value": round(cpu_tops, 6), "unit": "TOPS", "cores": 1,
                               "kind": "oracle", "sample": sample}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
