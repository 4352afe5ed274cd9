"""Seeded synthetic inputs for the N:M sparsification hot path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It draws random tensors and casts them to their storage dtype; it
holds none of the method's arithmetic (no score, no selection, no packing, no
matmul).

Recipe: numpy PCG64 seeded with ``SeedSequence([config_index, tensor_id])``;
every float tensor is drawn in float32 and then rounded to its storage dtype
(bfloat16 round-to-nearest-even via torch's CPU cast).  Shapes and value
distributions follow the five layer configurations the method is measured on:

* ``tiny24``     - 2:4 on a 256x256 fp32 layer with a per-column curvature vector.
* ``llama24``    - 2:4 bf16 on Llama-7B-shaped 4096x4096 / 11008x4096 layers with
                   1% outlier input channels scaled x20; calibration X 512x4096.
* ``slide68``    - 6:8 bf16 on a 14336x4096 FFN layer (SlideSparse's case).
* ``ternary68``  - 6:8 on a 6912x2560 ternary layer (Sparse-BitNet's case) with
                   int8 activations and per-token scales.
* ``hessian24``  - Hutchinson soft-mask step on a 28672x8192 bf16 layer with
                   calibration X 1024x8192.

All functions return CPU torch tensors; callers move them to the GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "rng", "normal_f32", "to_bf16", "CONFIGS", "Config",
    "tiny24_inputs", "llama24_weight", "llama24_calib", "activations_bf16",
    "slide68_weight", "ternary68_weights", "ternary68_activations",
    "hessian24_weight", "hessian24_calib", "TERNARY_TAU",
]


def rng(cfg: int, tensor_id: int) -> np.random.Generator:
    """Independent PCG64 stream for (config index, tensor id)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tensor_id])))


def normal_f32(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 ndarray -> bfloat16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    N: int
    M: int
    tokens: tuple = field(default_factory=tuple)


CONFIGS = {
    "tiny24": Config("tiny24", 0, 2, 4, (16,)),
    "llama24": Config("llama24", 1, 2, 4, (1, 16, 128, 2048)),
    "slide68": Config("slide68", 2, 6, 8, (1, 64, 512, 4096)),
    "ternary68": Config("ternary68", 3, 6, 8, (1, 256, 2048)),
    "hessian24": Config("hessian24", 4, 2, 4, (8192,)),
}

# Threshold giving P(|w| <= tau) = 0.42 for w ~ N(0,1): tau = Phi^-1(0.71).
TERNARY_TAU = 0.5533847195556729


# ---------------------------------------------------------------- tiny24 (config index 0)
def tiny24_inputs(R: int = 256, K: int = 256, tokens: int = 16):
    """W fp32 ~ 0.02 N(0,1); H fp32 ~ U(0.1, 1) per input column; X bf16 ~ N(0,1)."""
    W = torch.from_numpy(normal_f32(rng(0, 0), (R, K), 0.02))
    H = torch.from_numpy(rng(0, 1).uniform(0.1, 1.0, size=K).astype(np.float32))
    X = to_bf16(normal_f32(rng(0, 2), (tokens, K)))
    return W, H, X


# ---------------------------------------------------------------- llama24 (config index 1)
def llama24_outlier_columns(K: int = 4096, frac: float = 0.01) -> np.ndarray:
    n = int(math.ceil(frac * K))
    return np.sort(rng(1, 100).choice(K, size=n, replace=False))


def llama24_weight(R: int, K: int = 4096, tensor_id: int = 0) -> torch.Tensor:
    """bf16(0.02 N(0,1)) with ceil(1%) of the input columns scaled x20 (same column set for all layers)."""
    W = normal_f32(rng(1, tensor_id), (R, K), 0.02)
    W[:, llama24_outlier_columns(K)] *= np.float32(20.0)
    return to_bf16(W)


def llama24_calib(n: int = 512, K: int = 4096) -> torch.Tensor:
    return to_bf16(normal_f32(rng(1, 10), (n, K)))


def activations_bf16(cfg: int, tokens: int, K: int, tensor_id: int = 20) -> torch.Tensor:
    """Layer input X [tokens, K] bf16 ~ N(0,1)."""
    return to_bf16(normal_f32(rng(cfg, tensor_id + tokens), (tokens, K)))


def adapter_bf16(cfg: int, rank: int, K: int, R: int):
    """Stacked low-rank adapter pair of a layer: A [rank, K] ~ N(0,1)/sqrt(K) (down-
    projection) and B [R, rank] ~ 0.02 N(0,1) (up-projection), bf16."""
    A = to_bf16(normal_f32(rng(cfg, 40), (rank, K), 1.0 / np.sqrt(K)))
    B = to_bf16(normal_f32(rng(cfg, 41), (R, rank), 0.02))
    return A, B


# ---------------------------------------------------------------- slide68 (config index 2)
def slide68_weight(R: int = 14336, K: int = 4096) -> torch.Tensor:
    return to_bf16(normal_f32(rng(2, 0), (R, K), 0.02))


# ---------------------------------------------------------------- ternary68 (config index 3)
def ternary68_weights(R: int = 6912, K: int = 2560):
    """Latent bf16 master weights W_fp ~ N(0,1) and the ternary code W_t in {-1,0,+1}.

    W_t is drawn correlated with W_fp: zero where |W_fp| <= TERNARY_TAU (probability
    0.42), else sign(W_fp) (probability 0.29 each).  Returns (W_fp bf16, W_t int8).
    """
    Wf = to_bf16(normal_f32(rng(3, 0), (R, K)))
    a = Wf.float()
    Wt = torch.where(a.abs() > TERNARY_TAU, torch.sign(a), torch.zeros_like(a)).to(torch.int8)
    return Wf, Wt


def ternary68_activations(tokens: int, K: int = 2560):
    """X_q int8 ~ U{-127..127} and a positive per-token scale s_x (fp32)."""
    g = rng(3, 20 + tokens)
    Xq = torch.from_numpy(g.integers(-127, 128, size=(tokens, K), dtype=np.int8))
    sx = torch.from_numpy((g.uniform(0.5, 2.0, size=tokens) / 127.0).astype(np.float32))
    return Xq, sx


def ternary68_activations_bf16(tokens: int, K: int = 2560) -> torch.Tensor:
    """Unquantised activations for the int8 path: row m = a_m * U(-1, 1), a_m ~ U(0.5, 2), bf16."""
    g = rng(3, 40 + tokens)
    a = g.uniform(0.5, 2.0, size=(tokens, 1))
    return to_bf16((a * g.uniform(-1.0, 1.0, size=(tokens, K))).astype(np.float32))


# ---------------------------------------------------------------- hessian24 (config index 4)
def hessian24_weight(R: int = 28672, K: int = 8192) -> torch.Tensor:
    """W [out=R, in=K] bf16 ~ 0.015 N(0,1)."""
    return to_bf16(normal_f32(rng(4, 0), (R, K), 0.015))


def hessian24_calib(n: int = 1024, K: int = 8192) -> torch.Tensor:
    return to_bf16(normal_f32(rng(4, 10), (n, K)))


HESSIAN24_SEED = 4
HESSIAN24_PROBES = 8
HESSIAN24_EPS = 1e-6
HESSIAN24_T0 = 0.5
HESSIAN24_RHO = 0.5
HESSIAN24_STEPS = 8
