"""Query/key/value projection of the token matrix, plain float64 (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or call this module; the GPU library never does.

Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention" (German edition
of the self-attention / Triton / FlashAttention article, itimpress.au,
2026-11-15), §1:
  - the patches of an image form a token matrix X with N rows and D columns;
  - the first bullet ("Erzeugung von Queries, Keys und Values") forms three
    products of X with learned D x d_k matrices: Q = X W_Q, K = X W_K,
    V = X W_V;
  - the closing sentence of §1 runs attention in several heads side by side.

Readings where the article is silent:
  - each head h has its own W_Q, W_K, W_V; they are stored together in one
    weight array w[D, 3, H, d_k], where t = 0, 1, 2 selects Q, K, V;
  - the output is packed per token as qkv[B, N, 3, H, d_k]. That is the
    concatenated product X [W_Q | W_K | W_V] laid out for the attention's
    packed layout;
  - the formula has no bias term, and none is added;
  - a batch of B images shares the weights.
Backward: the calculus of the linear map, for a loss whose gradient with
respect to qkv is dqkv. It gives dX = dqkv W^T per token, and dW = X^T dqkv
summed over every token of the batch.

Pins that do not rest on this code live in tests/test_oracle_projection.py:
  - brute-force loops with math.fsum;
  - the closed form for identity weights;
  - finite differences;
  - the adjoint identity.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["qkv_projection", "qkv_projection_bwd", "brute_qkv_projection", "split_qkv"]


def _flat(x: np.ndarray, w: np.ndarray):
    if x.ndim != 3 or w.ndim != 4 or x.shape[2] != w.shape[0] or w.shape[1] != 3:
        raise ValueError("x must be [B, N, D] and w [D, 3, H, d_k]")
    B, N, D = x.shape
    return B, N, D, x.reshape(B * N, D), w.reshape(D, -1)


def qkv_projection(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """qkv[b, n, t, h, :] = x[b, n, :] @ w[:, t, h, :]  (§1: Q = X W_Q, K = X W_K, V = X W_V)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, N, D, x2, w2 = _flat(x, w)
    return (x2 @ w2).reshape((B, N) + w.shape[1:])


def qkv_projection_bwd(x: np.ndarray, w: np.ndarray, dqkv: np.ndarray):
    """(dx, dw) for a loss with gradient dqkv [B, N, 3, H, d_k] with respect to qkv.

    dx = dqkv W^T, one token row at a time. dw = X^T dqkv, with the sum running
    over all B * N tokens.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, N, D, x2, w2 = _flat(x, w)
    dy = np.asarray(dqkv, dtype=np.float64).reshape(B * N, w2.shape[1])
    dx = (dy @ w2.T).reshape(B, N, D)
    dw = (x2.T @ dy).reshape(w.shape)
    return dx, dw


def brute_qkv_projection(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """The same products as single dot products, one output entry at a time
    (math.fsum, no library matrix product). Pure Python, tiny shapes only."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, N, D = x.shape
    _, T, H, d = w.shape
    out = np.empty((B, N, T, H, d))
    for b in range(B):
        for n in range(N):
            for t in range(T):
                for h in range(H):
                    for j in range(d):
                        out[b, n, t, h, j] = math.fsum(float(x[b, n, c]) * float(w[c, t, h, j]) for c in range(D))
    return out


def split_qkv(qkv: np.ndarray):
    """Q, K, V as [B, H, N, d_k] arrays (copies) from a packed [B, N, 3, H, d_k] array."""
    return tuple(np.ascontiguousarray(qkv[:, :, t].transpose(0, 2, 1, 3)) for t in range(3))
