"""Shared plumbing for the GPU tests: upload seeded inputs, read results back, compare."""
from __future__ import annotations

import numpy as np

from attn_inputs import Inputs, bf16_bits_to_f64

# Tolerances. fp32 path: max-abs 1e-5 on O; bf16 inputs with fp32 accumulation:
# max-abs 2e-2 on O against the fp64 oracle run on the same bf16-rounded
# inputs; gradients: relative L2 error 5e-2 per tensor. lse (the saved row
# statistic): 1e-5 absolute for fp32; for 16-bit storage the per-row bound of
# lse_bound() below.
TOL_F32_O = 1e-5
TOL_F32_LSE = 1e-5
TOL_BF16_O = 2e-2
TOL_GRAD_RELL2 = 5e-2
# fp32 backward (fp32 storage and arithmetic): relative L2 1e-5 per gradient
# tensor, the fp32 forward's 1e-5 applied relative to the gradient's scale;
# every sum runs in fp32 over at most a few thousand terms (unit roundoff
# 6e-8), so the observed error sits near 1e-7.
TOL_F32_GRAD_RELL2 = 1e-5

U32 = 2.0 ** -24                             # fp32 unit roundoff
U_WEIGHT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}   # unit roundoff of the 16-bit weights


def term_rel_l2(got: np.ndarray, ref: np.ndarray, terms: np.ndarray) -> float:
    """||got - ref|| / ||terms||, with ``terms`` the same product taken over absolute values (for dQ = scale dS K:
    |scale| |dS| |K|). Rounding errors of a sum scale with the size of its terms, not with the sum, so where a
    gradient is a sum that cancels (rows of dS sum to 0), this is the measure the gradient tolerance applies to.
    Where nothing cancels it equals the relative L2 error."""
    den = float(np.linalg.norm(terms))
    return float(np.linalg.norm(got - ref)) / (den if den > 0 else 1.0)


def lse_bound(Q: np.ndarray, K: np.ndarray, scale: float, dtype: str, n_keys=None) -> np.ndarray:
    """Per-row bound on |lse_gpu - lse_exact| for 16-bit storage (fp32 accumulation).

    Q [..., M, d] and K [..., N, d] are the exact (16-bit) input values. The
    16-bit kernels compute lse = m + ln l with l the fp32 sum of the weights
    p_j = exp(s_j - m) rounded to the 16-bit type (the weights the P V product
    uses). The error terms, each a bound:
      weight rounding     each p_j off by at most u_w relative (round to nearest:
                          2^-8 for bf16, 2^-11 for fp16), so l by u_w relative
                          and ln l by u_w absolute;
      fp16 subnormals     fp16 weights below 2^-14 are rounded to multiples of
                          2^-24 (absolute error <= 2^-25 each); l >= 1 because
                          the largest weight is >= 1, so n * 2^-25;
      sum in fp32         a sum of n positive terms in any order, plus one
                          rescale per 32 keys at most: (n + n/32) * 2^-24;
      score in fp32       s_j = scale * sum_c q_c k_c: d exact products summed
                          in fp32, then the multiply by the fp32-rounded
                          scale * log2(e): |scale| * gamma * max_j sum_c
                          |q_c| |k_j,c| with gamma = (d + 2) u / (1 - (d + 2) u),
                          u = 2^-24; moving every exponent by at most that much
                          moves lse by at most that much;
      fp32 epilogue       the scale and ln 2 constants, m + log2 l and the
                          final multiply: a few ulps of |lse|, added by
                          lse_excess() as 2^-21 |lse|.
    With masks every row's visible keys are a subset of all N keys, so the
    bound over all keys still holds. n_keys defaults to K's row count.
    """
    d = Q.shape[-1]
    n = K.shape[-2] if n_keys is None else int(n_keys)
    gamma = (d + 2) * U32 / (1.0 - (d + 2) * U32)
    score = abs(scale) * gamma * np.matmul(np.abs(Q), np.swapaxes(np.abs(K), -1, -2)).max(axis=-1)
    t = U_WEIGHT[dtype] + (n + n / 32.0) * U32 + score
    if dtype == "f16":
        t = t + n * 2.0 ** -25
    return t


def lse_excess(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray) -> float:
    """Largest |gpu - ref| / (bound + 2^-21 |ref|) over finite reference rows; the check is lse_excess(...) <= 1.
    Rows whose reference is -inf (no visible key) must be -inf on the GPU too."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.broadcast_to(bound, ref.shape)
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), empty), "lse must be -inf exactly on the rows with no visible key"
    if not np.any(~empty):
        return 0.0
    g, r, b = gpu[~empty], ref[~empty], bound[~empty]
    return float(np.max(np.abs(g - r) / (b + 2.0 ** -21 * np.abs(r))))


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


def check_lse(gpu: np.ndarray, ref: np.ndarray, Q: np.ndarray, K: np.ndarray, scale: float, dtype: str,
              n_keys=None) -> float:
    """Assert the 16-bit lse is within lse_bound() of the oracle's; return the largest error / bound ratio."""
    e = lse_excess(gpu, ref, lse_bound(Q, K, scale, dtype, n_keys))
    assert e <= 1.0, f"lse error {e:.3f} x its bound"
    return e
