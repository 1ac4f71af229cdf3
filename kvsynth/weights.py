"""Seeded synthetic weights and activations for the weight-quantised decode GEMM.

Only random numbers, arranged into the GEMM's shapes: bf16 weight matrices [N][K] and bf16
activations [M][K] (one row per request being decoded).  No quantisation, scale or product is
computed here; the oracle and the GPU path both read these arrays.

The pages measure a whole model (GLM, weights in FP8 vs INT4, decode at 1..64 concurrent requests)
and give no layer shapes; the shapes below are stand-ins.  Weights are N(0, 0.02^2) -- the usual
order of magnitude of trained projection weights -- with a seeded 0.1% of the elements times 8, so
that groups differ in range and some groups' scales are set by a single large element.  Activations
are N(0, 1).  Draws use numpy.random.Generator(PCG64(SeedSequence([seed, tensor id, ...]))) and are
rounded to bf16 with torch's conversion, as for the KV cache inputs.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .workloads import _rng, bf16_bits_to_f32, to_bf16_bits

_T_W, _T_W_OUT, _T_X = 41, 42, 43


@dataclasses.dataclass(frozen=True)
class GemmShape:
    name: str
    n: int                   # output channels
    k: int                   # input channels
    layers: int = 1          # distinct weight matrices streamed per step
    seed: int = 0


def _shapes() -> dict:
    s = {}
    s["tiny"] = GemmShape("tiny", n=64, k=256, seed=0)
    s["ragged"] = GemmShape("ragged", n=320, k=1280, seed=1)
    s["wide"] = GemmShape("wide", n=4096, k=1280, seed=3)
    # a 16-matrix stack of 8192 x 8192 weights: 0.5 GB in INT4, 1 GB in FP8, so every step streams
    # from HBM (the 256 MB Infinity Cache cannot hold it)
    s["stack_8k"] = GemmShape("stack_8k", n=8192, k=8192, layers=16, seed=2)
    return s


SHAPES = _shapes()


def weights(shape: GemmShape, layer: int = 0, outlier_frac: float = 1e-3, outlier_mult: float = 8.0) -> np.ndarray:
    """bf16 bits [N][K] of one weight matrix."""
    w = _rng(shape.seed, _T_W, layer).standard_normal((shape.n, shape.k), dtype=np.float32) * np.float32(0.02)
    b = to_bf16_bits(w)
    if outlier_frac > 0:
        m = _rng(shape.seed, _T_W_OUT, layer).random((shape.n, shape.k)) < outlier_frac
        b[m] = to_bf16_bits(bf16_bits_to_f32(b[m]) * np.float32(outlier_mult))
    return b


def activations(shape: GemmShape, m: int, seed_offset: int = 0) -> np.ndarray:
    """bf16 bits [M][K]: one activation row per request."""
    x = _rng(shape.seed, _T_X, m, seed_offset).standard_normal((m, shape.k), dtype=np.float32)
    return to_bf16_bits(x)
