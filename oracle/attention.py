"""Plain fp64 CPU oracle for exact self-attention — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import or
call this module. The product library (HIP kernels behind the C ABI) neither
imports it nor shares any code, table or helper with it; the two meet only on
the seeded inputs from ``attn_inputs``.

Source. The article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention"
(German edition of the self-attention / Triton / FlashAttention article,
itimpress.au, 2026-11-15; the Telugu, Portuguese and Japanese editions carry the
same text):
  * §1, "Scores" formula: scores are the query-key dot products divided by
    sqrt(d_k); entry (i, j) says how much token i attends to token j.
  * §1, softmax paragraph: softmax is applied row by row, turning each row
    into probabilities that sum to 1; these weights multiply V.
  * §1, "Attention" formula: Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V.
  * §1, last paragraph: multi-head attention runs this same computation
    independently per head.
  * §3, recompute bullet: the forward keeps small per-row normalisation
    statistics; the backward rebuilds the attention tiles from them.

The oracle is the definition written out: it materialises the full score
matrix of one head at a time in float64, with no tiling, no online softmax and
no fusion. The kernel's scale is a free argument (the formula's 1/sqrt(d_k)
is what the workloads pass).

Readings where the article is silent:
  * Saved statistic = natural-log logsumexp of each scaled score row:
    lse_i = log(sum_j exp(s_ij)).
  * The softmax subtracts the row maximum before exponentiating. This is an
    exact identity (it cancels between numerator and denominator) and keeps
    exp() finite for the large scores of the stress workload.
  * The article prints no backward formulas. The gradients here are the
    calculus of the Attention formula for a scalar loss L with dL/dO = dO:
    dV = P^T dO, dP = dO V^T, dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
    (the Jacobian-vector product of the row softmax), dQ = scale * dS K,
    dK = scale * dS^T Q.

Array convention: q is [..., M, d], k and v are [..., N, d] with the same
leading (batch, head) dimensions; every leading index is an independent head.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

__all__ = [
    "attention_probs",
    "attention_fwd",
    "attention_bwd",
    "attention_ds",
    "brute_attention_fwd",
    "brute_attention_grads_fd",
]


def _heads(x: np.ndarray) -> np.ndarray:
    """View [..., rows, d] as [heads, rows, d]."""
    return x.reshape((-1,) + x.shape[-2:])


def _check(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> None:
    if q.ndim < 2 or k.ndim != q.ndim or v.ndim != q.ndim or not (q.shape[:-2] == k.shape[:-2] == v.shape[:-2]):
        raise ValueError(f"incompatible shapes q{q.shape} k{k.shape} v{v.shape}")
    if q.shape[-1] != k.shape[-1]:
        raise ValueError("q and k must share d_k")
    if k.shape[-2] != v.shape[-2]:
        raise ValueError("k and v must have the same number of rows")


def _head_probs(q: np.ndarray, k: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One head: the row-softmax of the scaled scores (§1 "Scores" and softmax paragraph).

    Returns (P [M, N], lse [M]).
    """
    s = (q @ k.T) * scale                      # scores: query-key dot products times the scale
    m = s.max(axis=1, keepdims=True)           # row maximum (exact shift, see module docstring)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l                                  # each row sums to 1
    lse = m[:, 0] + np.log(l[:, 0])            # natural-log logsumexp of the scaled row
    return p, lse


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """The full attention-probability matrix softmax(q k^T * scale), row-wise, per head."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    qh, kh = _heads(q), _heads(k)
    out = np.empty((qh.shape[0], qh.shape[1], kh.shape[1]), dtype=np.float64)
    for h in range(qh.shape[0]):
        out[h], _ = _head_probs(qh[h], kh[h], scale)
    return out.reshape(q.shape[:-1] + (k.shape[-2],))


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention(Q,K,V) = softmax(Q K^T * scale) V per head (§1 "Attention" formula).

    Returns (O [..., M, d_v], lse [..., M]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v)
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    o = np.empty((qh.shape[0], qh.shape[1], vh.shape[2]), dtype=np.float64)
    lse = np.empty(qh.shape[:2], dtype=np.float64)
    for h in range(qh.shape[0]):
        p, lse[h] = _head_probs(qh[h], kh[h], scale)
        o[h] = p @ vh[h]
    return o.reshape(q.shape[:-1] + (v.shape[-1],)), lse.reshape(q.shape[:-1])


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dQ, dK, dV) of L with dL/dO = do, for O = attention_fwd(q, k, v, scale)[0].

    P is rebuilt from the definition for each head (the oracle takes nothing
    from a forward pass). Calculus of the §1 "Attention" formula; see the
    module docstring.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _check(q, k, v)
    if do.shape != q.shape[:-1] + (v.shape[-1],):
        raise ValueError("do must have the shape of O")
    qh, kh, vh, doh = _heads(q), _heads(k), _heads(v), _heads(do)
    dq = np.empty_like(qh)
    dk = np.empty_like(kh)
    dv = np.empty_like(vh)
    for h in range(qh.shape[0]):
        p, ds = _head_ds(qh[h], kh[h], vh[h], doh[h], scale)
        dv[h] = p.T @ doh[h]                                   # dL/dV
        dq[h] = scale * (ds @ kh[h])                           # through the scores
        dk[h] = scale * (ds.T @ qh[h])
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


def _head_ds(q, k, v, do, scale):
    """One head: P and dS = dL/dS, the gradient with respect to the scaled scores (before the scale's chain
    rule): dP = dO V^T, dS = P * (dP - rowsum(P * dP)), the Jacobian-vector product of the row softmax."""
    p, _ = _head_probs(q, k, scale)
    dp = do @ v.T                                              # dL/dP
    rowdot = (p * dp).sum(axis=1, keepdims=True)               # sum_k P_ik dP_ik
    return p, p * (dp - rowdot)                                # through the row softmax


def attention_ds(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float) -> np.ndarray:
    """dS [..., M, N] of attention_bwd (dQ = scale dS K, dK = scale dS^T Q), per head."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    _check(q, k, v)
    qh, kh, vh, doh = _heads(q), _heads(k), _heads(v), _heads(do)
    out = np.empty((qh.shape[0], qh.shape[1], kh.shape[1]), dtype=np.float64)
    for h in range(qh.shape[0]):
        out[h] = _head_ds(qh[h], kh[h], vh[h], doh[h], scale)[1]
    return out.reshape(q.shape[:-1] + (k.shape[-2],))


# ----------------------------------------------------------------------------
# Brute force for tiny inputs: pure-Python loops straight from the formulas,
# sharing nothing with the vectorised oracle above.
# ----------------------------------------------------------------------------

def brute_attention_fwd(q, k, v, scale: float, allowed=None):
    """One head, pure Python: o_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij}, s_ij = scale * <q_i, k_j>.

    No max subtraction (inputs must keep scale*<q,k> small); sums use math.fsum.
    q: M x d, k: N x d, v: N x dv as nested sequences. Returns (o, lse) as lists.
    ``allowed`` (optional M x N booleans) drops the pairs it marks False from
    the sums; a row with no allowed pair gives o_i = 0 and lse_i = -inf.
    """
    q = [[float(x) for x in row] for row in q]
    k = [[float(x) for x in row] for row in k]
    v = [[float(x) for x in row] for row in v]
    o, lse = [], []
    for i, qi in enumerate(q):
        w = []
        for j, kj in enumerate(k):
            if allowed is not None and not allowed[i][j]:
                w.append(0.0)
                continue
            s = scale * math.fsum(a * b for a, b in zip(qi, kj))
            w.append(math.exp(s))
        z = math.fsum(w)
        if z == 0.0:
            o.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        o.append([math.fsum(w[j] * v[j][c] for j in range(len(k))) / z for c in range(len(v[0]))])
        lse.append(math.log(z))
    return o, lse


def brute_attention_grads_fd(q, k, v, do, scale: float, h: float = 1e-6, allowed=None):
    """Central finite differences of L = sum_ic O_ic * dO_ic through ``brute_attention_fwd``.

    Returns (dq, dk, dv) as float64 arrays. Only for tiny shapes.
    """
    q = np.array(q, dtype=np.float64)
    k = np.array(k, dtype=np.float64)
    v = np.array(v, dtype=np.float64)
    do = np.array(do, dtype=np.float64)

    def loss(qq, kk, vv):
        o, _ = brute_attention_fwd(qq.tolist(), kk.tolist(), vv.tolist(), scale, allowed)
        return math.fsum(o[i][c] * do[i, c] for i in range(len(o)) for c in range(len(o[0])))

    grads = []
    for which in range(3):
        base = [q, k, v]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(base[which].shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2.0 * h)
        grads.append(g)
    return tuple(grads)
