"""GPU parity of the memory layouts of attn_fwd_ex / attn_bwd_ex: token-major [B,N,H,d] and Q/K/V packed in
one [B,N,3,H,d] buffer (the output of one fused projection; the article's §1 forms Q, K and V from the patch
embeddings with three learned projections).

A layout changes only where rows are read and written, so every result must equal the [B,H,N,d] call bit for
bit (after the same transposition); one case per layout is also compared with the fp64 oracle.
"""
from __future__ import annotations

import sys

import pytest

from attn_inputs import make_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, max_abs, rel_l2, to_device, to_f64
from oracle import masked_attention_bwd, masked_attention_fwd

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(gpu_lib, layout, q, k, v, do, scale, causal, kv):
    """q, k, v, do given as [B, H, N, d]; returns O, lse, dQ, dK, dV as [B, H, N, d] (lse [B, H, N])."""
    import torch
    B, H, N, d = q.shape
    kvt = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    if layout == "bhnd":
        ins = (q, k, v)
        o, dob = torch.empty_like(q), do
        grads = tuple(torch.empty_like(q) for _ in range(3))
        back = lambda t: t
    else:
        tok = lambda t: t.transpose(1, 2).contiguous()                  # [B, N, H, d]
        if layout == "bnhd":
            ins = tuple(tok(t) for t in (q, k, v))
            gbuf = torch.empty((3, B, N, H, d), dtype=q.dtype, device="cuda")
            grads = tuple(gbuf[i] for i in range(3))
        else:
            packed = torch.stack([tok(t) for t in (q, k, v)], dim=2).contiguous()   # [B, N, 3, H, d]
            ins = tuple(packed[:, :, i] for i in range(3))
            gpk = torch.empty_like(packed)
            grads = tuple(gpk[:, :, i] for i in range(3))
        dob = tok(do)
        o = torch.empty((B, N, H, d), dtype=q.dtype, device="cuda")
        back = lambda t: t.transpose(1, 2)
    gpu_lib.attn_fwd_ex(*ins, o, lse, scale, causal=causal, kv_len=kvt, layout=layout)
    gpu_lib.attn_bwd_ex(*ins, o, lse, dob, *grads, scale, ws, causal=causal, kv_len=kvt, layout=layout)
    torch.cuda.synchronize()
    return (back(o).contiguous(), lse) + tuple(back(g).contiguous() for g in grads)


@pytest.mark.parametrize("layout", ["bnhd", "qkv_packed"])
@pytest.mark.parametrize("dtype,B,H,N,d,causal,kv", [
    ("bf16", 2, 3, 200, 64, False, None),
    ("bf16", 2, 2, 333, 128, True, [333, 100]),
    ("f16", 2, 2, 257, 32, True, None),
    ("bf16", 1, 4, 1100, 64, True, None),
    ("bf16", 2, 2, 1030, 96, False, [1030, 700]),
    ("bf16", 1, 3, 1030, 128, False, None),
    ("f16", 2, 2, 1100, 64, False, None),
])
def test_layout_matches_contiguous_bitwise(gpu_lib, layout, dtype, B, H, N, d, causal, kv):
    import torch
    x = make_case(B, H, N, d, dtype, seed=9000 + N + d)
    _say(f"layout {layout} {dtype} B={B} H={H} N={N} d={d} causal={causal} kv_len={kv}")
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    ref = _run(gpu_lib, "bhnd", q, k, v, do, x.scale, causal, kv)
    got = _run(gpu_lib, layout, q, k, v, do, x.scale, causal, kv)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("layout", ["bnhd", "qkv_packed"])
def test_layout_against_oracle(gpu_lib, layout):
    x = make_case(2, 3, 150, 64, "bf16", seed=9100)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o, lse, dq, dk, dv = _run(gpu_lib, layout, q, k, v, do, x.scale, True, [150, 77])
    Q, K, V, DO = x.f64("q"), x.f64("k"), x.f64("v"), x.f64("do")
    ro, _ = masked_attention_fwd(Q, K, V, x.scale, causal=True, kv_len=[150, 77])
    assert max_abs(to_f64(o), ro) <= TOL_BF16_O
    for got, r in zip((dq, dk, dv), masked_attention_bwd(Q, K, V, DO, x.scale, causal=True, kv_len=[150, 77])):
        assert rel_l2(to_f64(got), r) <= TOL_GRAD_RELL2


@pytest.mark.parametrize("B,H,N,fused", [(2, 3, 300, False), (2, 4, 196, True)])
def test_stages_equal_whole_backward(gpu_lib, B, H, N, fused):
    """attn_bwd_stage 0, 1, 2 in order equals attn_bwd_ex bit for bit (fp16, causal, key padding, packed layout),
    whether attn_bwd_ex launches the dK/dV and dQ work separately or as one kernel."""
    import torch
    assert gpu_lib.attn_bwd_fused(B, H, N, 64) == fused
    x = make_case(B, H, N, 64, "f16", seed=9200)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    tok = lambda t: t.transpose(1, 2).contiguous()
    packed = torch.stack([tok(t) for t in (q, k, v)], dim=2).contiguous()
    ins = tuple(packed[:, :, i] for i in range(3))
    dob = tok(do)
    kvt = torch.tensor([N, 123], dtype=torch.int32, device="cuda")
    o = torch.empty((B, N, H, d), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(*ins, o, lse, x.scale, causal=True, kv_len=kvt, layout="qkv_packed")
    outs = []
    for staged in (False, True):
        g = torch.full_like(packed, float("nan"))
        grads = tuple(g[:, :, i] for i in range(3))
        ws = gpu_lib.workspace_for(q)
        if staged:
            for st in (0, 1, 2):
                gpu_lib.attn_bwd_stage(st, *ins, o, lse, dob, *grads, x.scale, ws, causal=True, kv_len=kvt,
                                       layout="qkv_packed")
        else:
            gpu_lib.attn_bwd_ex(*ins, o, lse, dob, *grads, x.scale, ws, causal=True, kv_len=kvt, layout="qkv_packed")
        torch.cuda.synchronize()
        outs.append(g)
    assert torch.equal(outs[0], outs[1])
    assert torch.isfinite(outs[0].float()).all()
