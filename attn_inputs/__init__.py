"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it computes no part of
attention. Both the GPU path's callers (tests, bench) and the CPU oracle's
callers take their inputs from here, so the two sides always see identical
bits.

Workload shapes follow the article "Selbstaufmerksamkeit, CUDA-Kernel und
FlashAttention" (German edition of the self-attention / Triton / FlashAttention
article, itimpress.au, 2026-11-15): §1 gives the ViT token count N = 196
(224x224 image in 16x16 patches), width 768 and 12 heads, hence d_k = 64;
§3 motivates the long-sequence shapes (the N x N score matrix grows
quadratically with N).

Generator recipe (the same for every workload):
  rng = numpy.random.Generator(PCG64(SeedSequence([seed, workload_id])))
  draw order Q, K, V, dO; each drawn in float32 as rng.standard_normal * sigma
  (or rng.uniform(-1, 1) where the workload says so), then rounded
  round-to-nearest-even to bfloat16 for bf16 cases (to IEEE binary16 for f16
  cases, numpy's float16 conversion, also round-to-nearest-even). The rounded bits are
  uploaded unchanged, and their exact values (upcast to float64) feed the
  oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "Inputs",
    "make_inputs",
    "make_case",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "ProjInputs",
    "make_proj_case",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                 # "f32", "bf16" or "f16": storage type of Q, K, V, O, dO, dQ, dK, dV
    passes: Tuple[str, ...]    # ("fwd",) or ("fwd", "bwd")
    qk_sigma: float = 1.0      # Q, K ~ N(0, qk_sigma^2)
    v_dist: str = "normal"     # "normal" -> N(0,1); "uniform" -> U(-1, 1)
    planted_frac: float = 0.0  # fraction of query rows per head with a planted dominant key

    @property
    def scale(self) -> float:
        """1/sqrt(d_k) rounded to float32: the value handed to the kernel and the oracle alike."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The five workloads: the single-head fp32 case, the ViT-B/16 block, the long
# sequence, the very long sequence, and the online-softmax stress case.
WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "vit_single_head_fp32", 1, 1, 196, 64, "f32", ("fwd",)),
    2: Workload(2, "vit_b16_block", 32, 12, 196, 64, "bf16", ("fwd", "bwd")),
    3: Workload(3, "long_seq_4k", 8, 16, 4096, 64, "bf16", ("fwd", "bwd")),
    4: Workload(4, "very_long_seq_16k", 2, 16, 16384, 128, "bf16", ("fwd",)),
    5: Workload(5, "online_softmax_stress", 4, 12, 2048, 64, "bf16", ("fwd", "bwd"),
                qk_sigma=8.0, v_dist="uniform", planted_frac=0.01),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; return the uint16 bit patterns.

    Inputs here are finite (the generator draws no NaN/Inf).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


@dataclasses.dataclass
class Inputs:
    """One seeded problem instance.

    ``raw[name]`` holds what is uploaded: uint16 bit patterns for bf16 and f16
    cases, float32 for f32 ones, each of shape [B, H, N, d] contiguous.
    ``planted`` (stress workload only) is an int array [B, H, R, 2] of
    (query row, key row) pairs where K[key] was set to a copy of Q[row].
    """
    B: int
    H: int
    N: int
    d: int
    dtype: str
    scale: float
    raw: Dict[str, np.ndarray]
    planted: Optional[np.ndarray] = None

    def f64(self, name: str, index=...) -> np.ndarray:
        """Exact values of tensor ``name`` (optionally indexed first), as float64."""
        a = self.raw[name][index]
        if self.dtype == "bf16":
            return bf16_bits_to_f64(a)
        if self.dtype == "f16":
            return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
        return np.asarray(a, dtype=np.float64)


def _draw(rng: np.random.Generator, shape, dist: str, sigma: float) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        return x
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "ones":
        return np.ones(shape, dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_case(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0, wid: int = 0,
              qk_sigma: float = 1.0, v_dist: str = "normal", planted_frac: float = 0.0,
              with_grad: bool = True, scale: Optional[float] = None) -> Inputs:
    """Draw Q, K, V (and dO) for an arbitrary shape with the workload recipe."""
    if dtype not in ("bf16", "f16", "f32"):
        raise ValueError("dtype must be 'bf16', 'f16' or 'f32'")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(wid)])))
    shape = (B, H, N, d)
    q = _draw(rng, shape, "normal", qk_sigma)
    k = _draw(rng, shape, "normal", qk_sigma)
    v = _draw(rng, shape, v_dist, 1.0)
    do = _draw(rng, shape, "normal", 1.0) if with_grad else None

    planted = None
    R = int(round(planted_frac * N))
    if R > 0:
        # Per head: R distinct query rows and R distinct key rows, drawn without
        # replacement; key row j becomes an exact copy of query row i, so that
        # score (i, j) = |q_i|^2 * scale stands far above the rest of row i.
        planted = np.empty((B, H, R, 2), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                rows = rng.choice(N, size=R, replace=False)
                keys = rng.choice(N, size=R, replace=False)
                k[b, h, keys, :] = q[b, h, rows, :]
                planted[b, h, :, 0] = rows
                planted[b, h, :, 1] = keys

    raw = {}
    for name, arr in (("q", q), ("k", k), ("v", v), ("do", do)):
        if arr is None:
            continue
        if dtype == "bf16":
            raw[name] = f32_to_bf16_bits(arr).reshape(shape)
        elif dtype == "f16":
            raw[name] = arr.astype(np.float16).view(np.uint16)
        else:
            raw[name] = arr
    sc = float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale))
    return Inputs(B, H, N, d, dtype, sc, raw, planted)


def make_inputs(wid: int, seed: int = 0, with_grad: Optional[bool] = None) -> Inputs:
    """Inputs of workload ``wid`` (1..5) for ``seed``."""
    w = WORKLOADS[wid]
    if with_grad is None:
        with_grad = "bwd" in w.passes
    return make_case(w.B, w.H, w.N, w.d, w.dtype, seed=seed, wid=w.wid, qk_sigma=w.qk_sigma,
                     v_dist=w.v_dist, planted_frac=w.planted_frac, with_grad=with_grad)


@dataclasses.dataclass
class ProjInputs:
    """One seeded instance of the query/key/value projection that feeds attention.

    ``raw`` holds what is uploaded (uint16 bit patterns for "bf16" and "f16"):
      "x"    [B, N, D]          token matrix (§1: the N patch vectors of width D);
      "w"    [D, 3, H, d]       W_Q, W_K, W_V of every head side by side;
      "dqkv" [B, N, 3, H, d]    gradient with respect to the packed output.
    """
    B: int
    N: int
    D: int
    H: int
    d: int
    dtype: str
    raw: Dict[str, np.ndarray]

    def f64(self, name: str) -> np.ndarray:
        a = self.raw[name]
        if self.dtype == "bf16":
            return bf16_bits_to_f64(a)
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


def make_proj_case(B: int, N: int, D: int, H: int, d: int, dtype: str = "bf16", seed: int = 0,
                   wid: int = 0) -> ProjInputs:
    """Draw x ~ N(0, 1), w ~ N(0, 1/D) and dqkv ~ N(0, 1), in that order, rounded to ``dtype``.

    The weight spread 1/sqrt(D) keeps the projected values near unit size,
    the scale of the attention inputs the other workloads draw. The stream is
    PCG64(SeedSequence([seed, wid, 1])), separate from the attention inputs'.
    """
    if dtype not in ("bf16", "f16"):
        raise ValueError("dtype must be 'bf16' or 'f16'")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(wid), 1])))
    arrs = {
        "x": _draw(rng, (B, N, D), "normal", 1.0),
        "w": _draw(rng, (D, 3, H, d), "normal", float(1.0 / math.sqrt(D))),
        "dqkv": _draw(rng, (B, N, 3, H, d), "normal", 1.0),
    }
    raw = {}
    for name, arr in arrs.items():
        if dtype == "bf16":
            raw[name] = f32_to_bf16_bits(arr).reshape(arr.shape)
        else:
            raw[name] = arr.astype(np.float16).view(np.uint16)
    return ProjInputs(B, N, D, H, d, dtype, raw)
