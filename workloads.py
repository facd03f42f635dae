"""Seeded synthetic inputs for the block-wise INT8 linear and its grouped MoE form.

Shared by the oracle's tests and the GPU path's tests and benchmark, and by
nothing else.  It holds none of the method's arithmetic: it draws random
numbers, stores them in the caller's dtypes and lays them out.  Quantisation,
scale shapes and every GEMM live elsewhere (the oracle or the HIP library).

Value distributions (the shapes are the workloads the block-INT8 linear is
measured on; no dataset or trained weight is involved):

* activations: fp32 N(0, 1), optionally a fraction of channels (columns)
  multiplied by an outlier factor, then stored as bf16 (one RNE rounding done
  by torch's dtype conversion);
* int8 weights: uniform on [-127, 127];
* fp32 weight block scales: exp(N(-6, 0.5)) (log-normal, median ~2.5e-3);
* MoE router logits: fp32 N(0, 1); tokens are dispatched to their top-k
  experts by logit (equal to top-k by softmax probability), and the dispatched
  rows are ordered by (expert, token, slot).
"""
from __future__ import annotations

import numpy as np
import torch

# The measured workloads, by name.  ``seed`` is the generator seed; the MLP
# pair and the ragged case share one seed family (sub-seeds differ).
CONFIGS = {
    "tiny":    dict(seed=(0, 0), M=16, K=256, N=256),
    "decode":  dict(seed=(1, 0), M=8, K=4096, N=4096, outlier_frac=0.01, outlier_scale=20.0),
    "prefill": dict(seed=(2, 0), M=4096, K=4096, N=4096),
    "gate_up": dict(seed=(3, 0), M=2048, K=4096, N=28672),
    "down":    dict(seed=(3, 1), M=2048, K=14336, N=4096),
    "ragged":  dict(seed=(3, 2), M=333, K=4000, N=5000),
    "moe":     dict(seed=(4, 0), T=4096, H=4096, I=14336, E=8, topk=2),
}


def rng_for(seed) -> np.random.Generator:
    return np.random.default_rng(list(seed) if isinstance(seed, (tuple, list)) else seed)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store an fp32 array as bf16 bits (uint16), via torch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def activations(rng, M: int, K: int, outlier_frac: float = 0.0,
                outlier_scale: float = 20.0) -> np.ndarray:
    """bf16 bits [M, K]: N(0,1), with round(outlier_frac*K) columns scaled."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out > 0:
        cols = rng.choice(K, n_out, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    return to_bf16_bits(x)


def weights(rng, *shape) -> np.ndarray:
    """int8 uniform on [-127, 127]."""
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def weight_scales(rng, *shape) -> np.ndarray:
    """fp32 log-normal exp(N(-6, 0.5)) of the given (block-scale) shape."""
    return np.exp(rng.normal(-6.0, 0.5, size=shape)).astype(np.float32)


def router_logits(rng, T: int, E: int) -> np.ndarray:
    return rng.standard_normal((T, E), dtype=np.float32)
