"""Shared plumbing for the GPU tests: upload seeded inputs, read results back, compare."""
from __future__ import annotations

import numpy as np

from attn_inputs import Inputs, bf16_bits_to_f64

# Tolerances. fp32 path: max-abs 1e-5 on O; bf16 inputs with fp32 accumulation:
# max-abs 2e-2 on O against the fp64 oracle run on the same bf16-rounded
# inputs; gradients: relative L2 error 5e-2 per tensor. lse (the saved row
# statistic): 1e-5 absolute for fp32; for bf16 inputs 4e-3 * max(1, |lse|):
# the kernels normalise by the sum of the bf16-rounded weights (the weights the
# P V product uses), each off by at most 2^-8 relative (round to nearest, 8
# significant bits), so l is off by at most 2^-8 relative and lse = m + ln l by
# at most 2^-8 ~ 3.9e-3 absolute; rows with few visible keys (causal mask)
# come close to that bound because their rounding errors do not average out.
TOL_F32_O = 1e-5
TOL_F32_LSE = 1e-5
TOL_BF16_O = 2e-2
TOL_BF16_LSE_REL = 4e-3
TOL_GRAD_RELL2 = 5e-2
# fp16 storage: the same O and gradient bounds; the weights carry 11
# significant bits (at most 2^-11 ~ 4.9e-4 relative rounding), so lse is held
# to 1e-3 * max(1, |lse|).
TOL_F16_LSE_REL = 1e-3
# fp32 backward (fp32 storage and arithmetic): relative L2 1e-5 per gradient
# tensor, the fp32 forward's 1e-5 applied relative to the gradient's scale;
# every sum runs in fp32 over at most a few thousand terms (unit roundoff
# 6e-8), so the observed error sits near 1e-7.
TOL_F32_GRAD_RELL2 = 1e-5


def to_device(x: Inputs, name: str):
    import torch
    a = x.raw[name]
    if x.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_f64(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (den if den > 0 else 1.0)


def lse_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest |gpu - ref| / max(1, |ref|)."""
    return float(np.max(np.abs(gpu - ref) / np.maximum(1.0, np.abs(ref)))) if gpu.size else 0.0
