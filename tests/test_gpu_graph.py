"""HIP graph capture of the whole path (attn_fwd_ex + attn_bwd_ex, three backward launches), and of the ViT block
with its query/key/value projection: every replay must equal the eager results bit for bit. The kernels record no
memset and no host synchronisation, so a captured step is just its kernel launches. Replays are interleaved with
other eager work and synchronisations.
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


def test_graph_vit_block_with_projection(gpu_lib):
    """The ViT attention block with its query/key/value projection captured as one graph: projection, attention
    in the packed layout, attention backward and projection backward (whose dx product splits its contraction,
    so the split-sum kernel is captured too). Every replay equals the eager results bit for bit."""
    import numpy as np
    import torch
    from attn_inputs import make_proj_case
    B, N, D, H, d = 4, 196, 768, 12, 64
    c = make_proj_case(B, N, D, H, d, "bf16", seed=77)
    g = make_case(B, H, N, d, "bf16", seed=77)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    x, w = up(c.raw["x"]), up(c.raw["w"])
    do = up(g.raw["do"]).transpose(1, 2).contiguous()
    qkv = torch.empty((B, N, 3, H, d), dtype=torch.bfloat16, device="cuda")
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dqkv = torch.empty_like(qkv)
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    ws = torch.empty(gpu_lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    pws = gpu_lib.proj_workspace_for(x, w)
    assert pws is not None                                   # the dx product splits at this size
    outs = (qkv, o, lse, dqkv, dx, dw)

    def step():
        gpu_lib.attn_qkv_proj(x, w, qkv)
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, g.scale, layout="qkv_packed")
        gpu_lib.attn_bwd_ex(q, k, v, o, lse, do, dqkv[:, :, 0], dqkv[:, :, 1], dqkv[:, :, 2], g.scale, ws,
                            layout="qkv_packed")
        gpu_lib.attn_qkv_proj_bwd(x, w, dqkv, dx, dw, pws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outs + (pws,):
            t.fill_(float("nan") if t.is_floating_point() else 255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("qkv", "o", "lse", "dqkv", "dx", "dw"), outs, eager):
            assert torch.equal(a, b), f"replay {rep}: {name}"
        _ = (x.float() @ x.float().transpose(-1, -2)).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
