"""Masked attention: plain fp64 CPU definition — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import or
call this module; the GPU library shares nothing with it.

The article ("Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention", §1
"Attention" formula) defines unmasked attention only. §3 opens with long text
sequences as the case where the N x N score matrix becomes the limit; for text
two masks are standard, and this module is the reading taken for them (the
article prints neither):
  * key padding: batch entry b holds kv_len[b] real keys; keys j >= kv_len[b]
    take no part in any row of that entry;
  * causal: query i sees keys j <= i only (positions counted from 0 in the
    same sequence as the keys).
A masked pair gets score -inf, i.e. probability 0; the softmax of each row runs
over its visible keys only. A row with no visible key has an empty sum: its
output is 0, its logsumexp is -inf (log 0) and it passes no gradient.

Arrays: q [B, H, M, d], k and v [B, H, N, d], do [B, H, M, d_v]; kv_len is None
(all N keys) or B integers in [0, N]; q_index gives the sequence position of
each of the M query rows (default 0..M-1), so that a few rows of a long
sequence can be checked against the full keys.
"""
from __future__ import annotations

import numpy as np

__all__ = ["visible_keys", "masked_attention_fwd", "masked_attention_bwd", "masked_attention_dq_rows",
           "masked_attention_ds"]


def visible_keys(N: int, q_index, causal: bool, kv_len_b: int) -> np.ndarray:
    """Boolean [M, N]: entry (r, j) is True when query row r (at position q_index[r]) sees key j."""
    j = np.arange(N)[None, :]
    vis = j < int(kv_len_b)
    if causal:
        vis = vis & (j <= np.asarray(q_index)[:, None])
    return np.broadcast_to(vis, (len(q_index), N)).copy()


def _lengths(B: int, N: int, kv_len):
    if kv_len is None:
        return [N] * B
    kv = [int(x) for x in kv_len]
    if len(kv) != B or min(kv) < 0 or max(kv) > N:
        raise ValueError("kv_len needs B entries in [0, N]")
    return kv


def _masked_probs(qh, kh, scale, vis):
    """One head: P [M, N] over the visible keys, lse [M]; rows with no visible key give P = 0, lse = -inf."""
    s = np.where(vis, (qh @ kh.T) * scale, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1), 0.0)                # row max over visible keys (0 for empty rows)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return p, lse


def masked_attention_fwd(q, k, v, scale: float, causal: bool = False, kv_len=None, q_index=None):
    """O_i = sum over visible j of softmax_j(scale <q_i, k_j>) v_j, per (b, h). Returns (O, lse) in float64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    if q.ndim != 4 or k.shape[:2] != q.shape[:2] or v.shape[:3] != k.shape[:3] or q.shape[3] != k.shape[3]:
        raise ValueError(f"shapes q{q.shape} k{k.shape} v{v.shape}")
    B, H, M, _ = q.shape
    N = k.shape[2]
    qi = np.arange(M) if q_index is None else np.asarray(q_index)
    kv = _lengths(B, N, kv_len)
    o = np.zeros((B, H, M, v.shape[3]))
    lse = np.empty((B, H, M))
    for b in range(B):
        vis = visible_keys(N, qi, causal, kv[b])
        for h in range(H):
            p, lse[b, h] = _masked_probs(q[b, h], k[b, h], scale, vis)
            o[b, h] = p @ v[b, h]
    return o, lse


def masked_attention_bwd(q, k, v, do, scale: float, causal: bool = False, kv_len=None):
    """Gradients (dQ, dK, dV) of sum(O * dO) for O = masked_attention_fwd(...) over all N query rows.

    Same calculus as the unmasked oracle, with P = 0 on masked pairs:
    dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = scale dS K, dK = scale dS^T Q.
    """
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, M, _ = q.shape
    N = k.shape[2]
    if M != N:
        raise ValueError("the backward takes every query row of the sequence")
    kv = _lengths(B, N, kv_len)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        vis = visible_keys(N, np.arange(M), causal, kv[b])
        for h in range(H):
            p, _ = _masked_probs(q[b, h], k[b, h], scale, vis)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def masked_attention_dq_rows(q, k, v, do, scale: float, causal: bool = False, kv_len=None, q_index=None):
    """dQ of the M query rows given (at sequence positions q_index), for the loss sum(O * dO) over those rows.

    Row i of dQ depends on row i alone: dS_i = P_i * (dP_i - sum_j P_ij dP_ij) with dP_i = dO_i V^T, and
    dQ_i = scale dS_i K (the same calculus as masked_attention_bwd, restricted to the given rows), so a few
    rows of a long sequence can be checked without the full N x N matrices. q, do: [B, H, M, d]; k, v:
    [B, H, N, d]."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, M, _ = q.shape
    N = k.shape[2]
    qi = np.arange(M) if q_index is None else np.asarray(q_index)
    kv = _lengths(B, N, kv_len)
    dq = np.empty_like(q)
    for b in range(B):
        vis = visible_keys(N, qi, causal, kv[b])
        for h in range(H):
            p, _ = _masked_probs(q[b, h], k[b, h], scale, vis)
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, h])
    return dq


def masked_attention_ds(q, k, v, do, scale: float, causal: bool = False, kv_len=None):
    """dS [B, H, N, N] of masked_attention_bwd (dQ = scale dS K, dK = scale dS^T Q): the gradient with respect to
    the scaled scores, 0 on masked pairs."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, M, _ = q.shape
    N = k.shape[2]
    if M != N:
        raise ValueError("dS takes every query row of the sequence")
    kv = _lengths(B, N, kv_len)
    out = np.empty((B, H, M, N))
    for b in range(B):
        vis = visible_keys(N, np.arange(M), causal, kv[b])
        for h in range(H):
            p, _ = _masked_probs(q[b, h], k[b, h], scale, vis)
            dp = do[b, h] @ v[b, h].T
            out[b, h] = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return out
