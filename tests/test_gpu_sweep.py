"""Seeded random sweep of the extended entry points (attn_fwd_ex / attn_bwd_ex) against the masked fp64 oracle.

Each case draws, from one fixed-seed generator:
  - storage type (bf16, fp16), layout ([B,H,N,d], [B,N,H,d], packed [B,N,3,H,d]) and head dim (32, 64, 96, 128);
  - a ragged sequence length N, batch B and heads H;
  - the causal mask on or off, and per-entry key lengths kv_len (including 0 and N) or none;
  - the scale: 1/sqrt(d), a larger or a negative multiple, or 0 (uniform weights).
Every case checks the forward (O, lse, rows with no visible key) and the backward (relative L2 per gradient, exact
zeros where the masks force them) at the same tolerances as the fixed-shape tests. The fixed shapes elsewhere
cover the workloads' sizes; this sweep covers combinations they do not.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from attn_inputs import make_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, check_lse, max_abs, rel_l2, to_device, to_f64
from oracle import masked_attention_bwd, masked_attention_fwd

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([32, 64, 96, 128]))
        N = int(rng.choice([1, 2, 31, 33, 64, 65, 127, 196, 255, 300, 513, 700]))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        kv = None
        if rng.integers(0, 2):
            kv = [int(rng.choice([0, 1, N, max(1, N // 2), int(rng.integers(0, N + 1))])) for _ in range(B)]
        mult = float(rng.choice([1.0, 2.5, -1.0, 0.0]))
        out.append(dict(i=i, dtype=str(rng.choice(["bf16", "f16"])), layout=str(rng.choice(["bhnd", "bnhd", "qkv_packed"])),
                        B=B, H=H, N=N, d=d, causal=causal, kv=kv, mult=mult))
    return out


def _run(gpu_lib, layout, q, k, v, do, scale, causal, kv):
    """q, k, v, do as [B, H, N, d]; returns O, lse, dQ, dK, dV as [B, H, N, d] (lse [B, H, N])."""
    import torch
    B, H, N, d = q.shape
    kvt = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    if layout == "bhnd":
        ins, dob = (q, k, v), do
        o = torch.empty_like(q)
        grads = tuple(torch.empty_like(q) for _ in range(3))
        back = lambda t: t
    else:
        tok = lambda t: t.transpose(1, 2).contiguous()
        if layout == "bnhd":
            ins = tuple(tok(t) for t in (q, k, v))
            gb = torch.empty((3, B, N, H, d), dtype=q.dtype, device="cuda")
            grads = tuple(gb[i] for i in range(3))
        else:
            packed = torch.stack([tok(t) for t in (q, k, v)], dim=2).contiguous()
            ins = tuple(packed[:, :, i] for i in range(3))
            gp = torch.empty_like(packed)
            grads = tuple(gp[:, :, i] for i in range(3))
        dob = tok(do)
        o = torch.empty((B, N, H, d), dtype=q.dtype, device="cuda")
        back = lambda t: t.transpose(1, 2)
    gpu_lib.attn_fwd_ex(*ins, o, lse, scale, causal=causal, kv_len=kvt, layout=layout)
    gpu_lib.attn_bwd_ex(*ins, o, lse, dob, *grads, scale, ws, causal=causal, kv_len=kvt, layout=layout)
    torch.cuda.synchronize()
    return (to_f64(back(o).contiguous()), lse.cpu().numpy().astype(np.float64)) + \
        tuple(to_f64(back(g).contiguous()) for g in grads)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c['i']}")
def test_random_case_against_oracle(gpu_lib, case):
    c = case
    print(f"[sweep] {c}", flush=True)
    sys.stdout.flush()
    x = make_case(c["B"], c["H"], c["N"], c["d"], c["dtype"], seed=7000 + c["i"])
    scale = float(np.float32(c["mult"] * x.scale))
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = _run(gpu_lib, c["layout"], q, k, v, do, scale, c["causal"], c["kv"])
    Q, K, V, DO = x.f64("q"), x.f64("k"), x.f64("v"), x.f64("do")
    ro, rl = masked_attention_fwd(Q, K, V, scale, causal=c["causal"], kv_len=c["kv"])
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), "rows with no visible key must give lse = -inf"
    assert np.all(o[empty] == 0)
    assert max_abs(o, ro) <= TOL_BF16_O
    check_lse(lse, rl, Q, K, scale, c["dtype"])
    ref = masked_attention_bwd(Q, K, V, DO, scale, causal=c["causal"], kv_len=c["kv"])
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert rel_l2(g, r) <= TOL_GRAD_RELL2, name
    if c["kv"] is not None:
        for b, n in enumerate(c["kv"]):
            assert np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0)
            if n == 0:
                assert np.all(dq[b] == 0)
    if scale == 0.0:
        # Uniform weights: S carries no gradient, so dQ and dK vanish exactly.
        assert np.all(dq == 0) and np.all(dk == 0)
