"""Seeded synthetic inputs for row-major GEMV (no GEMV arithmetic here).

This module only draws random operands.  It serves both the HIP path and the
CPU oracle, and holds none of either side's arithmetic: no products, no
dequantisation, no packing of values chosen elsewhere.

Workloads (all synthetic; no page uses a dataset):
  f32 : A and x i.i.d. uniform[-1, 1], cast to float32 (round to nearest even)
        -- the square FP32 study of "cuda-gemv-optimization".
  f16 : A ~ N(0, 1/N), x ~ N(0, 1), cast to binary16 -- decode-projection
        shapes from "membound", section "Results".
  f16x32 : A ~ N(0, 1/N) as binary16, x ~ N(0, 1) kept in float32 (FP16
        weights with an FP32 hidden state, as the llama.cpp original keeps it).
  f16_acc16 : the f16 operands (the lossy FP16-accumulation entry point).
  q8  : A int8 uniform on [-127, 127]; one binary16 scale per row,
        uniform[0.5, 1.5]/127; x ~ N(0, 1) binary16.
  q4  : A packed two nibbles per byte, [M, N/2] uint8.  Every byte is drawn
        uniform on 0..255, so each nibble is independently uniform over its
        16 codes, i.e. uniform on [-8, 7] read as two's complement; one
        binary16 scale per row and 128-column group, uniform[0.5, 1.5]/7,
        stored [M, N/128]; x ~ N(0, 1) binary16.
Every shape draws from numpy's PCG64 ``default_rng(seed)`` afresh, in the
order A, scales, x.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

KINDS = ("f32", "f16", "f16x32", "f16_acc16", "q8", "q4")


@dataclass(frozen=True)
class Workload:
    kind: str
    M: int
    N: int

    @property
    def name(self) -> str:
        return f"{self.kind}_{self.M}x{self.N}"


# The workload families, at their full sizes.
WORKLOADS = {
    "f32_1024": [Workload("f32", 1024, 1024)],
    "f32_sweep": [Workload("f32", n, n) for n in (2048, 4096, 8192)],
    "f16_decode": [Workload("f16", 4096, 4096), Workload("f16", 8192, 8192),
                   Workload("f16", 14336, 4096), Workload("f16", 4096, 14336)],
    "q8_decode": [Workload("q8", 8192, 8192), Workload("q8", 14336, 4096)],
    "f16x32_decode": [Workload("f16x32", 8192, 8192), Workload("f16x32", 4096, 14336)],
    "f16_acc16_decode": [Workload("f16_acc16", 8192, 8192), Workload("f16_acc16", 4096, 14336)],
    "q4_decode": [Workload("q4", 4096, 14336), Workload("q4", 14336, 4096)],
}


def all_workloads():
    return [w for ws in WORKLOADS.values() for w in ws]


def make_f32(M: int, N: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1.0, 1.0, (M, N)).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, N).astype(np.float32)
    return {"A": A, "x": x}


def make_f16(M: int, N: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    sigma = 1.0 / np.sqrt(N) if N > 0 else 1.0
    A = rng.normal(0.0, sigma, (M, N)).astype(np.float16)
    x = rng.standard_normal(N).astype(np.float16)
    return {"A": A, "x": x}


def make_f16x32(M: int, N: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    sigma = 1.0 / np.sqrt(N) if N > 0 else 1.0
    A = rng.normal(0.0, sigma, (M, N)).astype(np.float16)
    x = rng.standard_normal(N).astype(np.float32)
    return {"A": A, "x": x}


def make_q8(M: int, N: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    A = rng.integers(-127, 128, (M, N), dtype=np.int8)
    scale = rng.uniform(0.5 / 127.0, 1.5 / 127.0, M).astype(np.float16)
    x = rng.standard_normal(N).astype(np.float16)
    return {"A": A, "scale": scale, "x": x}


def make_q4(M: int, N: int, seed: int = 0):
    if N % 128 != 0:
        raise ValueError("INT4 rows are made of whole 128-column groups (N % 128 == 0)")
    rng = np.random.default_rng(seed)
    A = rng.integers(0, 256, (M, N // 2), dtype=np.uint8)
    scale = rng.uniform(0.5 / 7.0, 1.5 / 7.0, (M, N // 128)).astype(np.float16)
    x = rng.standard_normal(N).astype(np.float16)
    return {"A": A, "scale": scale, "x": x}


def make_weights(M: int, N: int, seed: int = 0) -> np.ndarray:
    """FP32 weights uniform on [-1, 1]: the quantiser's input, the
    distribution on which the "membound" page reports its quantisation RMSE."""
    rng = np.random.default_rng(seed)
    return rng.uniform(-1.0, 1.0, (M, N)).astype(np.float32)


# Activation distributions beyond the workloads' zero-mean N(0, 1): decode
# hidden states after an activation are non-negative or off-centre.
X_DISTS = ("normal", "abs_normal", "shifted")


def make_x_f16(N: int, dist: str = "normal", seed: int = 0) -> np.ndarray:
    """binary16 x: ``normal`` N(0, 1), ``abs_normal`` |N(0, 1)|, ``shifted``
    N(1, 1)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(N)
    if dist == "normal":
        v = z
    elif dist == "abs_normal":
        v = np.abs(z)
    elif dist == "shifted":
        v = z + 1.0
    else:
        raise ValueError(f"unknown x distribution {dist!r}")
    return v.astype(np.float16)


def make_gauss_weights(M: int, N: int, seed: int = 0, outlier: float = 0.0) -> np.ndarray:
    """FP32 weights ~ N(0, 1), the quantiser's input for realistic codes.  With
    ``outlier`` > 0 one weight per row (at a random column) is set to that
    value, so that the row's absmax scale leaves most codes small."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((M, N)).astype(np.float32)
    if outlier > 0 and N > 0:
        W[np.arange(M), rng.integers(0, N, M)] = np.float32(outlier)
    return W


# Quantiser workloads: the INT8 and INT4 GEMV shapes, from FP32 weights.
QUANT_WORKLOADS = [("q8", 8192, 8192), ("q8", 14336, 4096), ("q4", 4096, 14336), ("q4", 14336, 4096)]


def make_logits(M: int, N: int, seed: int = 0) -> np.ndarray:
    """Softmax input: binary16 logits ~ N(0, 1) (the page does not print its
    distribution; the GEMV's own x recipe is reused)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, N)).astype(np.float16)


# Softmax workloads: the row shapes of the "membound" softmax table.
SOFTMAX_WORKLOADS = [(8192, 8192), (4096, 32768), (1024, 131072)]


MAKERS = {"f32": make_f32, "f16": make_f16, "f16x32": make_f16x32, "f16_acc16": make_f16, "q8": make_q8,
          "q4": make_q4}


def make(kind: str, M: int, N: int, seed: int = 0):
    return MAKERS[kind](M, N, seed)
