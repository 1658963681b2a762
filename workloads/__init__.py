"""Seeded synthetic inputs for the NVFP4 linear-layer workloads.

This module holds random draws and shapes only -- none of the method's
arithmetic -- and is the one piece that both the oracle side (tests, the CPU
baseline) and the GPU side (tests, bench.py) use.

Recipe (the pages train on web-scale text; no dataset or trained weight is used
here, these draws stand in for the activations, weights and gradients of the
pages' 12B / 3B / 1.9B models):
  * one numpy.random.default_rng(seed) per workload, tensors drawn in the order
    listed, in float32, then rounded to bfloat16 (nearest-even) where the
    workload is bf16;
  * activations X ~ N(0, 1) (the fprop workload adds outliers: exactly
    floor(0.001 * numel) distinct positions, chosen uniformly without
    replacement by the same generator, multiplied by 50);
  * weights W ~ N(0, 0.02^2);
  * output gradients dY ~ Laplace(0, 1e-3);
  * the random-Hadamard sign mask is the low 16 bits of the next uint32 drawn
    after the tensors; stochastic rounding uses seed 0 with offset 1 for dgrad's
    dY and offset 2 for wgrad's dY.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

SR_SEED = 0
SR_OFFSET_DGRAD = 1
SR_OFFSET_WGRAD = 2


def normal(rng: np.random.Generator, shape, std=1.0, outlier_frac=0.0, outlier_scale=50.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_frac > 0.0:
        n = int(np.floor(outlier_frac * x.size))
        idx = rng.choice(x.size, size=n, replace=False)
        x.reshape(-1)[idx] *= np.float32(outlier_scale)
    return x


def error_operands(M: int, N: int, K: int, seed: int, outliers: bool):
    """Operands of the error-versus-K analysis, drawn in this order: A [M, K] like
    activations (N(0, 1), with 0.1% of the entries x50 when `outliers`), B [N, K]
    like weights (N(0, 0.02^2)), then the 16-bit Hadamard sign mask; both rounded
    to bf16."""
    rng = np.random.default_rng(seed)
    a = normal(rng, (M, K), outlier_frac=0.001 if outliers else 0.0)
    b = normal(rng, (N, K), std=0.02)
    signs = int(rng.integers(0, 2**32, dtype=np.uint64)) & 0xFFFF
    return to_bf16(a), to_bf16(b), signs


def laplace(rng: np.random.Generator, shape, scale=1e-3) -> np.ndarray:
    return rng.laplace(0.0, scale, size=shape).astype(np.float32)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bfloat16 torch CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def widen(t: torch.Tensor) -> np.ndarray:
    """bfloat16/float32 torch CPU tensor -> float32 numpy (exact)."""
    return t.float().numpy()


@dataclass
class Linear:
    """One linear layer y = x . w^T: M tokens, K input features, N output features."""
    name: str
    M: int
    N: int
    K: int


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    linears: list
    x_outliers: bool = False
    passes: tuple = ("fprop", "dgrad", "wgrad")
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", torch.float32, [Linear("tiny", 256, 256, 256)], passes=("fprop",),
                     description="X, W 256x256 fp32 ~ N(0,1), 1D nearest-even, Y = X.W^T fp32"),
    "fprop_8k": Workload("fprop_8k", torch.bfloat16, [Linear("fprop", 8192, 4096, 4096)], x_outliers=True,
                         passes=("fprop",),
                         description="X 8192x4096 ~ N(0,1) with 0.1% x50 outliers, W 4096x4096 ~ N(0,0.02^2) 2D"),
    "wgrad_8k": Workload("wgrad_8k", torch.bfloat16, [Linear("wgrad", 8192, 4096, 4096)], passes=("wgrad",),
                         description="dY 8192x4096 ~ Laplace(0,1e-3), X 8192x4096 ~ N(0,1), RHT+SR, dW fp32"),
    "mlp_up_12b": Workload("mlp_up_12b", torch.bfloat16, [Linear("mlp_up", 16384, 20480, 5120)],
                           description="12B-hybrid-like MLP up-projection: X 16384x5120, W 20480x5120, "
                                       "dY 16384x20480; fprop + dgrad + wgrad"),
    "block_3b": Workload("block_3b", torch.bfloat16,
                         [Linear("qkv", 32768, 9216, 3072), Linear("o", 32768, 3072, 3072),
                          Linear("up", 32768, 8192, 3072), Linear("down", 32768, 3072, 8192)],
                         description="3B-like block linears at 32768 tokens: fprop + dgrad + wgrad of all four"),
}


@dataclass
class LinearInputs:
    x: torch.Tensor          # [M, K] CPU
    w: torch.Tensor          # [N, K] CPU
    dy: Optional[torch.Tensor]  # [M, N] CPU (None when the workload has no backward)
    signs: int


def make_linear_inputs(lin: Linear, dtype=torch.bfloat16, seed=0, x_outliers=False, with_dy=True) -> LinearInputs:
    """Draw X, W, dY (in that order) and then the sign mask from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (lin.M, lin.K), outlier_frac=0.001 if x_outliers else 0.0)
    w = normal(rng, (lin.N, lin.K), std=0.02)
    dy = laplace(rng, (lin.M, lin.N)) if with_dy else None
    signs = int(rng.integers(0, 2**32, dtype=np.uint64)) & 0xFFFF
    cast = (lambda a: to_bf16(a)) if dtype == torch.bfloat16 else (lambda a: torch.from_numpy(a))
    return LinearInputs(cast(x), cast(w), None if dy is None else cast(dy), signs)


def make_tiny(seed=0):
    """The tiny case: X then W, fp32 N(0,1), from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((256, 256), dtype=np.float32)
    w = rng.standard_normal((256, 256), dtype=np.float32)
    return torch.from_numpy(x), torch.from_numpy(w)


def random_matrix(shape, seed, kind="normal", std=1.0, dtype=torch.bfloat16) -> torch.Tensor:
    """A single seeded matrix for parity cases of other shapes."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        a = normal(rng, shape, std=std)
    elif kind == "laplace":
        a = laplace(rng, shape, scale=std)
    elif kind == "outliers":
        a = normal(rng, shape, std=std, outlier_frac=0.001)
    else:
        raise ValueError(kind)
    return to_bf16(a) if dtype == torch.bfloat16 else torch.from_numpy(a)
