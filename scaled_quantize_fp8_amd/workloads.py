"""Seeded synthetic inputs and layer shapes of the FP8 linear workloads.

This module holds no quantization or GEMM arithmetic: it only names shapes
and draws seeded random tensors on the host (fp32 normal draws times sigma,
rounded once to bf16), so the HIP path and the CPU oracle can be fed the
same bytes.

Seeds: seed_t = 1000 * seed + tensor_id + 16 * linear_index, tensor ids
X=1, W=2, bias=3, G=4, outlier mask=5, drift=6.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

TENSOR_IDS = {"X": 1, "W": 2, "bias": 3, "G": 4, "outlier": 5, "drift": 6}


def seed_for(seed: int, tensor: str, linear_index: int = 0) -> int:
    return 1000 * seed + TENSOR_IDS[tensor] + 16 * linear_index


def _gen(seed_t: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_t)
    return g


def normal_bf16(shape, sigma: float, seed_t: int) -> torch.Tensor:
    """bf16 CPU tensor: fp32 N(0,1) draws times sigma, rounded to bf16."""
    x = torch.randn(tuple(shape), generator=_gen(seed_t), dtype=torch.float32)
    return (x * sigma).to(torch.bfloat16)


def normal_with_outliers_bf16(shape, sigma: float, seed_x: int, seed_mask: int,
                              p: float = 1e-3, factor: float = 50.0) -> torch.Tensor:
    """N(0, sigma) draws where an iid Bernoulli(p) mask multiplies by factor,
    then rounded to bf16 (activations with 0.1% outliers x50)."""
    x = torch.randn(tuple(shape), generator=_gen(seed_x), dtype=torch.float32) * sigma
    mask = torch.rand(tuple(shape), generator=_gen(seed_mask)) < p
    x = torch.where(mask, x * factor, x)
    return x.to(torch.bfloat16)


def log_uniform_drift(steps: int, seed_t: int, lo: float = -2.0, hi: float = 2.0) -> list[float]:
    """iid d_t with log10 d_t ~ U[lo, hi] (amax drift of the pre-quantized
    workload)."""
    u = torch.rand(steps, generator=_gen(seed_t), dtype=torch.float64)
    return [float(10.0 ** (lo + (hi - lo) * v)) for v in u]


# --------------------------------------------------------------------------
# Layer shapes.  (name, K = in_features, N = out_features)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Linear:
    name: str
    K: int
    N: int


TINY = [Linear("tiny", 256, 256)]
DIM1024 = [Linear("qkv", 1024, 3072), Linear("out", 1024, 1024),
           Linear("up", 1024, 4096), Linear("down", 4096, 1024)]
DIM1536 = [Linear("qkv", 1536, 4608), Linear("out", 1536, 1536),
           Linear("up", 1536, 6912), Linear("gate", 1536, 6912),
           Linear("down", 6912, 1536)]
GENERIC = [Linear("w1", 4096, 11008), Linear("w2", 11008, 4096)]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    linears: tuple
    sigma_x: float
    sigma_w: float
    sigma_g: float
    sigma_b: float
    outliers: bool
    delayed: bool          # ring (delayed scaling) vs dynamic
    hist_len: int


WORKLOADS = {
    "tiny": Workload("tiny", 128, tuple(TINY), 1.0, 0.02, 1e-3, 0.01, False, True, 16),
    "dim1024_m2048": Workload("dim1024_m2048", 2048, tuple(DIM1024), 1.0, 0.02, 1e-3, 0.01,
                              False, True, 16),
    "dim1536_m2048": Workload("dim1536_m2048", 2048, tuple(DIM1536), 1.0, 0.02, 1e-3, 0.01,
                              True, True, 16),
    "dim1536_m512": Workload("dim1536_m512", 512, tuple(DIM1536), 1.0, 0.02, 1e-3, 0.01,
                             True, True, 16),
    "generic_m4096": Workload("generic_m4096", 4096, tuple(GENERIC), 1.0, 0.015, 1e-4, 0.01,
                              False, False, 16),
    "prequant_dim1536_m2048": Workload("prequant_dim1536_m2048", 2048, tuple(DIM1536), 1.0,
                                       0.02, 1e-3, 0.01, False, True, 16),
}

# multipliers of X over the four steps of the tiny workload
TINY_STEP_FACTORS = (1.0, 4.0, 0.25, 16.0)
PREQUANT_STEPS = 8


def layer_inputs(wl: Workload, li: int, seed: int = 0, M: int | None = None):
    """bf16 CPU tensors (X [M,K], W [N,K], bias [N], G [M,N]) of linear li."""
    lin = wl.linears[li]
    M = wl.M if M is None else M
    if wl.outliers:
        X = normal_with_outliers_bf16((M, lin.K), wl.sigma_x, seed_for(seed, "X", li),
                                      seed_for(seed, "outlier", li))
    else:
        X = normal_bf16((M, lin.K), wl.sigma_x, seed_for(seed, "X", li))
    W = normal_bf16((lin.N, lin.K), wl.sigma_w, seed_for(seed, "W", li))
    b = normal_bf16((lin.N,), wl.sigma_b, seed_for(seed, "bias", li))
    G = normal_bf16((M, lin.N), wl.sigma_g, seed_for(seed, "G", li))
    return X, W, b, G
