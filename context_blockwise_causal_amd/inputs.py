"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This module holds no attention arithmetic: it only draws numbers and rounds them to the
storage dtype.  Both the HIP path and the FP64 oracle receive exactly the arrays made here.

Recipe (one draw per workload):
  * ``numpy.random.Generator(PCG64(seed))``;
  * ``standard_normal`` in float32, full-sequence B,H,S,D order, drawn in the order
    Q (B,Hq,S,D), K (B,Hkv,S,D), V (B,Hkv,S,D), dO (B,Hq,S,D);
  * bf16 workloads then round every float32 to bf16 with round-to-nearest-even, done here
    with integer bit arithmetic so that it does not depend on any library's conversion.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite normal draws; NaN and Inf are not expected and not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensors:
    """One workload's tensors.

    ``store`` holds what the device receives (float32 arrays, or uint16 bf16 bit patterns);
    ``as_f64(name)`` gives the exact same values widened to float64 for the oracle.
    """

    dtype: str  # "f32" or "bf16"
    store: dict

    def as_f32(self, name: str) -> np.ndarray:
        a = self.store[name]
        if self.dtype == "bf16":
            return f32_from_bf16_bits(a)
        return a

    def as_f64(self, name: str) -> np.ndarray:
        return self.as_f32(name).astype(np.float64)


def draw(batch: int, seq_len: int, heads_q: int, heads_kv: int, head_dim: int, dtype: str,
         seed: int, with_grad: bool = True) -> Tensors:
    """Draw Q, K, V (and dO) for a full-sequence problem per the recipe in the module doc."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = [("q", (batch, heads_q, seq_len, head_dim)),
              ("k", (batch, heads_kv, seq_len, head_dim)),
              ("v", (batch, heads_kv, seq_len, head_dim))]
    if with_grad:
        shapes.append(("do", (batch, heads_q, seq_len, head_dim)))
    store = {}
    for name, shape in shapes:
        x = rng.standard_normal(size=shape, dtype=np.float32)
        store[name] = bf16_bits_from_f32(x) if dtype == "bf16" else x
    return Tensors(dtype=dtype, store=store)


def draw_like(shape, dtype: str, seed: int) -> np.ndarray:
    """One extra N(0,1) tensor (store form) for unit tests of single entry points."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x
