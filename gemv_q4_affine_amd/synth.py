"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random tensors of the workloads' shapes and nothing else:
it holds none of the quantisation or matmul arithmetic, so that the CPU oracle
and the HIP path can both be fed from it without sharing any of the method.

Recipe (numpy PCG64, ``default_rng(seed)``):
  * weights  W = standard_normal((N, K)) * 0.02, cast to float32;
  * activations X = standard_normal((M, K)), cast to float32;
  * bfloat16 inputs are the round-to-nearest-even bfloat16 of those float32
    values (the MLX repro casts its normal draws to bfloat16 the same way).
The weights are drawn first, then the activations, from one generator.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def weights(rng: np.random.Generator, N: int, K: int, scale: float = 0.02) -> np.ndarray:
    return (rng.standard_normal((N, K)) * scale).astype(np.float32)


def activations(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    return rng.standard_normal((M, K)).astype(np.float32)


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    K: int
    M: int
    seed: int = 0


# The workloads of the pages, with their shapes.
TINY = Workload("q4_0 tiny", N=256, K=512, M=4, seed=0)
DECODE = Workload("decode gemv q4_0 x q8_1", N=12288, K=4096, M=1, seed=0)
PREFILL = Workload("prefill gemm q4_0 bf16", N=12288, K=4096, M=2048, seed=0)
AFFINE_MS = (1, 32, 512, 2048, 8192)
AFFINE = Workload("affine4 g64 sweep", N=12288, K=4096, M=0, seed=0)

# Llama-3.2-1B-shaped projection shapes (N, K) per layer, 16 layers.
LLAMA1B_LAYERS = 16
LLAMA1B_SHAPES = {
    "q": (2048, 2048),
    "k": (512, 2048),
    "v": (512, 2048),
    "o": (2048, 2048),
    "gate": (8192, 2048),
    "up": (8192, 2048),
    "down": (2048, 8192),
}


def workload_inputs(w: Workload, M: int | None = None):
    """(W float32 [N,K], X float32 [M,K]) for a workload, weights drawn first."""
    rng = np.random.default_rng(w.seed)
    W = weights(rng, w.N, w.K)
    X = activations(rng, w.M if M is None else M, w.K)
    return W, X
