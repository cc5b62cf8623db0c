"""HIP graph capture of the whole path (attn_fwd_ex + attn_bwd_ex, three backward launches): every replay must
equal the eager results bit for bit. The kernels record no memset and no host synchronisation, so a captured
step is just the four kernel launches. Replays are interleaved with other eager work and synchronisations.
"""
from __future__ import annotations

import pytest

from attn_inputs import make_case
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
def test_graph_replays_equal_eager(gpu_lib, causal):
    import torch
    x = make_case(4, 12, 196, 64, "bf16", seed=321)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = gpu_lib.workspace_for(q)

    def step():
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, causal=causal)
        gpu_lib.attn_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, x.scale, ws, causal=causal)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a side stream, as graph capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), eager):
            assert torch.equal(a, b), f"replay {rep}: {name}"
        _ = (q.float() @ k.float().transpose(-1, -2)).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
