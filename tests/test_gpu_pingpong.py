"""The 16-bit forward kernels agree bit for bit, and so do the two dK/dV kernels.

Unmasked rows of 1024 keys or more at d_k = 128 run the ping-pong forward,
and unmasked rows of whole 64-key tiles (256 keys or more) at d_k = 64 the
software-pipelined forward; both compute the same tiles with the same
arithmetic per element as the single-phase forward, in another order. A
key-padding length equal to N hides no key but routes the same inputs to the
single-phase kernel, so the results must be identical (O and lse): bf16 and
fp16, contiguous and packed layouts, and (pipelined forward) inputs whose
scores are large enough that many tiles take its full rescale path; causal
rows (pipelined tiles, then the diagonal) likewise. All are
also checked against the fp64 oracle by the parity tests.
"""
from __future__ import annotations

import sys

import pytest

from attn_inputs import make_case
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,B,H,N,layout", [
    ("bf16", 1, 2, 1024, "bhnd"), ("bf16", 2, 1, 1100, "bhnd"), ("bf16", 1, 2, 2047, "bhnd"),
    ("f16", 1, 2, 1300, "bhnd"), ("bf16", 2, 2, 1030, "qkv_packed"),
])
def test_pingpong_equals_single_phase(gpu_lib, dtype, B, H, N, layout):
    import torch
    d = 128
    x = make_case(B, H, N, d, dtype, seed=7000 + N)
    print(f"pingpong {dtype} B={B} H={H} N={N} d={d} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v = (to_device(x, n) for n in ("q", "k", "v"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        if layout == "qkv_packed":
            o = torch.empty((B, N, H, d), dtype=q.dtype, device="cuda")
        else:
            o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, kv_len=kv, layout=layout)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]), "O"
    assert torch.equal(outs[0][1], outs[1][1]), "lse"


@pytest.mark.parametrize("dtype,B,H,N,sigma,layout", [
    ("bf16", 1, 2, 256, 1.0, "bhnd"), ("bf16", 2, 3, 320, 1.0, "bhnd"), ("f16", 1, 2, 1024, 1.0, "bhnd"),
    ("bf16", 1, 4, 4096, 1.0, "bhnd"), ("bf16", 2, 3, 2048, 8.0, "bhnd"), ("f16", 1, 2, 576, 8.0, "bhnd"),
    ("bf16", 2, 2, 512, 1.0, "qkv_packed"),
])
def test_pipelined_equals_single_phase(gpu_lib, dtype, B, H, N, sigma, layout):
    import torch
    d = 64
    x = make_case(B, H, N, d, dtype, seed=7100 + N, qk_sigma=sigma, with_grad=False)
    print(f"pipelined {dtype} B={B} H={H} N={N} d={d} sigma={sigma} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v = (to_device(x, n) for n in ("q", "k", "v"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        o = torch.empty((B, N, H, d) if layout == "qkv_packed" else (B, H, N, d), dtype=q.dtype, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, kv_len=kv, layout=layout)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype,B,H,N,sigma,layout", [
    ("bf16", 1, 2, 256, 1.0, "bhnd"), ("bf16", 2, 3, 384, 1.0, "bhnd"), ("f16", 1, 2, 1152, 1.0, "bhnd"),
    ("bf16", 1, 4, 4096, 1.0, "bhnd"), ("bf16", 2, 3, 2048, 8.0, "bhnd"), ("bf16", 2, 2, 640, 1.0, "qkv_packed"),
])
def test_pipelined_dkdv_causal_equals_single_phase(gpu_lib, dtype, B, H, N, sigma, layout):
    """Causal rows of whole 128-key blocks at d_k = 64 run the software-pipelined dK/dV kernel from each block's
    first visible step, its first two steps masked (the diagonal); a key-padding length equal to N routes the same
    inputs to the single-phase kernel: dK and dV must be identical. The stage is called on its own."""
    import torch
    d = 64
    x = make_case(B, H, N, d, dtype, seed=7500 + N, qk_sigma=sigma)
    print(f"pipelined causal dK/dV {dtype} B={B} H={H} N={N} d={d} sigma={sigma} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        do = do.permute(0, 2, 1, 3).contiguous()
    shape = (B, N, H, d) if layout == "qkv_packed" else (B, H, N, d)
    o = torch.empty(shape, dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, causal=True, layout=layout)
    ws = gpu_lib.workspace_for(q)

    def grads():  # dQ, dK, dV filled with NaN (slices of one packed buffer for the packed layout)
        if layout == "qkv_packed":
            g = torch.full((B, N, 3, H, d), float("nan"), dtype=q.dtype, device="cuda")
            return g[:, :, 0], g[:, :, 1], g[:, :, 2]
        return tuple(torch.full(shape, float("nan"), dtype=q.dtype, device="cuda") for _ in range(3))

    gpu_lib.attn_bwd_stage(0, q, k, v, o, lse, do, *grads(), x.scale, ws, causal=True, layout=layout)
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        dq, dk, dv = grads()
        gpu_lib.attn_bwd_stage(1, q, k, v, o, lse, do, dq, dk, dv, x.scale, ws, causal=True, kv_len=kv,
                               layout=layout)
        outs.append((dk, dv))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0][0].float()).all()) and bool(torch.isfinite(outs[0][1].float()).all())
    assert torch.equal(outs[0][0], outs[1][0]), "dK"
    assert torch.equal(outs[0][1], outs[1][1]), "dV"


@pytest.mark.parametrize("dtype,B,H,N,sigma,layout", [
    ("bf16", 1, 2, 256, 1.0, "bhnd"), ("bf16", 2, 3, 320, 1.0, "bhnd"), ("bf16", 1, 2, 576, 1.0, "bhnd"),
    ("f16", 1, 2, 1088, 1.0, "bhnd"), ("bf16", 1, 4, 4096, 1.0, "bhnd"), ("bf16", 2, 3, 2048, 8.0, "bhnd"),
    ("bf16", 2, 2, 704, 1.0, "qkv_packed"),
    # ragged last steps: rows past N read as row N - 1 and masked
    ("bf16", 2, 3, 196, 1.0, "bhnd"), ("bf16", 1, 2, 129, 1.0, "bhnd"), ("f16", 2, 2, 1000, 8.0, "bhnd"),
    ("bf16", 2, 2, 197, 1.0, "qkv_packed"),
])
def test_pipelined_dkdv_equals_single_phase(gpu_lib, dtype, B, H, N, sigma, layout):
    """Unmasked rows of at least three 64-query steps (the last may be partial) at d_k = 64 run the
    software-pipelined dK/dV kernel; a key-padding length equal to N routes the same inputs to the single-phase
    kernel, which performs the same operations per element in the same order: dK and dV must be identical. The
    stage is called on its own, so that the fused dK/dV + dQ launch of small grids does not take over."""
    import torch
    d = 64
    x = make_case(B, H, N, d, dtype, seed=7200 + N, qk_sigma=sigma)
    print(f"pipelined dK/dV {dtype} B={B} H={H} N={N} d={d} sigma={sigma} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        do = do.permute(0, 2, 1, 3).contiguous()
    shape = (B, N, H, d) if layout == "qkv_packed" else (B, H, N, d)
    o = torch.empty(shape, dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, layout=layout)
    ws = gpu_lib.workspace_for(q)

    def grads():  # dQ, dK, dV filled with NaN (slices of one packed buffer for the packed layout)
        if layout == "qkv_packed":
            g = torch.full((B, N, 3, H, d), float("nan"), dtype=q.dtype, device="cuda")
            return g[:, :, 0], g[:, :, 1], g[:, :, 2]
        return tuple(torch.full(shape, float("nan"), dtype=q.dtype, device="cuda") for _ in range(3))

    gpu_lib.attn_bwd_stage(0, q, k, v, o, lse, do, *grads(), x.scale, ws, layout=layout)
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        dq, dk, dv = grads()
        gpu_lib.attn_bwd_stage(1, q, k, v, o, lse, do, dq, dk, dv, x.scale, ws, kv_len=kv, layout=layout)
        outs.append((dk, dv))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0][0].float()).all()) and bool(torch.isfinite(outs[0][1].float()).all())
    assert torch.equal(outs[0][0], outs[1][0]), "dK"
    assert torch.equal(outs[0][1], outs[1][1]), "dV"


@pytest.mark.parametrize("dtype,B,H,N,sigma,layout", [
    ("bf16", 2, 3, 256, 1.0, "bhnd"), ("bf16", 4, 12, 2048, 8.0, "bhnd"), ("f16", 2, 2, 1088, 1.0, "bhnd"),
    ("bf16", 2, 3, 196, 1.0, "bhnd"), ("bf16", 1, 2, 129, 1.0, "bhnd"), ("bf16", 2, 2, 1000, 8.0, "qkv_packed"),
])
def test_pipelined_dq_equals_single_phase(gpu_lib, dtype, B, H, N, sigma, layout):
    """Small unmasked grids at d_k = 64 (at least three 64-key tiles, the last may be partial) run the
    software-pipelined dQ kernel; a key-padding length equal to N routes the same inputs to the single-phase
    kernel, which sums the same products in the same order: dQ must be identical."""
    import torch
    d = 64
    x = make_case(B, H, N, d, dtype, seed=7400 + N, qk_sigma=sigma)
    print(f"pipelined dQ {dtype} B={B} H={H} N={N} d={d} sigma={sigma} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        do = do.permute(0, 2, 1, 3).contiguous()
    shape = (B, N, H, d) if layout == "qkv_packed" else (B, H, N, d)
    o = torch.empty(shape, dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, layout=layout)
    ws = gpu_lib.workspace_for(q)

    def grads():
        if layout == "qkv_packed":
            g = torch.full((B, N, 3, H, d), float("nan"), dtype=q.dtype, device="cuda")
            return g[:, :, 0], g[:, :, 1], g[:, :, 2]
        return tuple(torch.full(shape, float("nan"), dtype=q.dtype, device="cuda") for _ in range(3))

    gpu_lib.attn_bwd_stage(0, q, k, v, o, lse, do, *grads(), x.scale, ws, layout=layout)
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        dq, dk, dv = grads()
        gpu_lib.attn_bwd_stage(2, q, k, v, o, lse, do, dq, dk, dv, x.scale, ws, kv_len=kv, layout=layout)
        outs.append(dq)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0].float()).all())
    assert torch.equal(outs[0], outs[1]), "dQ"


@pytest.mark.parametrize("dtype,B,H,N,layout", [
    ("bf16", 2, 4, 196, "bhnd"), ("f16", 4, 2, 256, "bhnd"), ("bf16", 2, 4, 1000, "bhnd"), ("bf16", 2, 4, 197, "qkv_packed"),
])
def test_combined_pipelined_launch_equals_stages(gpu_lib, dtype, B, H, N, layout):
    """Where the combined dK/dV + dQ launch applies and the rows are unmasked, it runs the pipelined dK/dV body
    (ragged last step masked) beside the dQ body: stage 3 must give dQ, dK, dV identical to stages 1 and 2."""
    import torch
    d = 64
    assert gpu_lib.attn_bwd_fused(B, H, N, d)
    x = make_case(B, H, N, d, dtype, seed=7300 + N)
    print(f"combined pipelined launch {dtype} B={B} H={H} N={N} layout={layout}", flush=True)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        do = do.permute(0, 2, 1, 3).contiguous()
    shape = (B, N, H, d) if layout == "qkv_packed" else (B, H, N, d)
    o = torch.empty(shape, dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, layout=layout)
    ws = gpu_lib.workspace_for(q)

    def grads():
        if layout == "qkv_packed":
            g = torch.full((B, N, 3, H, d), float("nan"), dtype=q.dtype, device="cuda")
            return g, (g[:, :, 0], g[:, :, 1], g[:, :, 2])
        g = torch.full((3,) + shape, float("nan"), dtype=q.dtype, device="cuda")
        return g, (g[0], g[1], g[2])

    gpu_lib.attn_bwd_stage(0, q, k, v, o, lse, do, *grads()[1], x.scale, ws, layout=layout)
    outs = []
    for stages in ((1, 2), (3,)):
        g, g3 = grads()
        for st in stages:
            gpu_lib.attn_bwd_stage(st, q, k, v, o, lse, do, *g3, x.scale, ws, layout=layout)
        outs.append(g)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[1].float()).all())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("d,dtype,B,H,N,sigma,layout", [
    (128, "bf16", 1, 2, 1024, 1.0, "bhnd"), (128, "bf16", 2, 2, 2048, 1.0, "bhnd"),
    (128, "f16", 2, 1, 1088, 1.0, "bhnd"), (128, "bf16", 1, 2, 4096, 8.0, "bhnd"),
    (128, "bf16", 2, 2, 1152, 1.0, "qkv_packed"),
    (64, "bf16", 1, 2, 1024, 1.0, "bhnd"), (64, "bf16", 2, 3, 2048, 8.0, "bhnd"), (64, "f16", 2, 2, 1088, 1.0, "bhnd"),
    (64, "bf16", 1, 2, 4096, 1.0, "bhnd"), (64, "bf16", 2, 2, 1152, 1.0, "qkv_packed"),
])
def test_pipelined_causal_equals_single_phase(gpu_lib, d, dtype, B, H, N, sigma, layout):
    """Causal rows of whole 64-key tiles (1024 keys or more) at d_k = 64 and 128 run the pipelined forward on the
    tiles a workgroup's queries see in full, then the diagonal tiles with the single-phase kernel's masked tile; a
    key-padding length of N routes the same inputs to the single-phase kernel: O and lse must be identical
    (N = 1088 and 1152 end in a partial row block; sigma 8 gives peaked scores)."""
    import torch
    x = make_case(B, H, N, d, dtype, seed=7400 + N + d, qk_sigma=sigma, with_grad=False)
    print(f"pipelined causal d={d} {dtype} B={B} H={H} N={N} sigma={sigma} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v = (to_device(x, n) for n in ("q", "k", "v"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        o = torch.empty((B, N, H, d) if layout == "qkv_packed" else (B, H, N, d), dtype=q.dtype, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, causal=True, kv_len=kv, layout=layout)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0][1]).all())
    assert torch.equal(outs[0][0], outs[1][0]), "O"
    assert torch.equal(outs[0][1], outs[1][1]), "lse"


@pytest.mark.parametrize("dtype,B,H,N,sigma,layout", [
    ("bf16", 1, 2, 1024, 1.0, "bhnd"), ("bf16", 2, 2, 2048, 1.0, "bhnd"), ("f16", 2, 1, 1088, 1.0, "bhnd"),
    ("bf16", 1, 2, 4096, 8.0, "bhnd"), ("bf16", 2, 2, 1152, 1.0, "qkv_packed"),
])
def test_pipelined128_equals_single_phase(gpu_lib, dtype, B, H, N, sigma, layout):
    """Unmasked rows of whole 64-key tiles (1024 keys or more) at d_k = 128 run the software-pipelined forward with
    one query block per wave; a key-padding length of N routes the same inputs to the single-phase kernel: O and lse
    must be identical (including peaked scores, whose units take the maximum-first path)."""
    import torch
    d = 128
    x = make_case(B, H, N, d, dtype, seed=7300 + N, qk_sigma=sigma, with_grad=False)
    print(f"pipelined d=128 {dtype} B={B} H={H} N={N} sigma={sigma} layout={layout}", flush=True)
    sys.stdout.flush()
    q, k, v = (to_device(x, n) for n in ("q", "k", "v"))
    if layout == "qkv_packed":
        qkv = torch.stack([q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)], dim=2).contiguous()
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        o = torch.empty((B, N, H, d) if layout == "qkv_packed" else (B, H, N, d), dtype=q.dtype, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, kv_len=kv, layout=layout)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]), "O"
    assert torch.equal(outs[0][1], outs[1][1]), "lse"


# Causal rows on the pipelined kernels over grid shapes: head counts whose work splits evenly over the 8 XCDs or
# not (the two branches of the heaviest-first order), lengths at and past the thresholds, partial last row blocks.
CAUSAL_SWEEP = [(d, B, H, N) for d in (64, 128) for (B, H) in ((1, 1), (1, 3), (3, 5), (2, 4))
                for N in (1024, 1088, 1344, 2112)]


@pytest.mark.parametrize("d,B,H,N", CAUSAL_SWEEP)
def test_causal_pipelined_forward_sweep(gpu_lib, d, B, H, N):
    """The pipelined causal forward equals the single-phase kernel (key padding of N) bit for bit."""
    import torch
    x = make_case(B, H, N, d, "bf16", seed=7600 + N + d + B * H, with_grad=False)
    print(f"causal sweep fwd d={d} B={B} H={H} N={N}", flush=True)
    sys.stdout.flush()
    q, k, v = (to_device(x, n) for n in ("q", "k", "v"))
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, causal=True, kv_len=kv)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0][1]).all())
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("B,H,N", [(B, H, N) for (B, H) in ((1, 1), (1, 3), (3, 5), (2, 4)) for N in (256, 384, 1152, 2048)])
def test_causal_pipelined_dkdv_sweep(gpu_lib, B, H, N):
    """The pipelined causal dK/dV kernel equals the single-phase kernel (key padding of N) bit for bit."""
    import torch
    d = 64
    x = make_case(B, H, N, d, "bf16", seed=7700 + N + B * H)
    print(f"causal sweep dK/dV B={B} H={H} N={N}", flush=True)
    sys.stdout.flush()
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, causal=True)
    ws = gpu_lib.workspace_for(q)
    grads = lambda: tuple(torch.full_like(q, float("nan")) for _ in range(3))
    gpu_lib.attn_bwd_stage(0, q, k, v, o, lse, do, *grads(), x.scale, ws, causal=True)
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    outs = []
    for kv in (None, full):
        dq, dk, dv = grads()
        gpu_lib.attn_bwd_stage(1, q, k, v, o, lse, do, dq, dk, dv, x.scale, ws, causal=True, kv_len=kv)
        outs.append((dk, dv))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0][0].float()).all())
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
