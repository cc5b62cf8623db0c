"""GPU parity of the query/key/value projection (attn_qkv_proj / attn_qkv_proj_bwd) with the fp64 oracle.

Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention", §1 first bullet: Q = X W_Q, K = X W_K,
V = X W_V with one set of D x d_k weights per head. The kernels compute each output as a float32 sum of exact
16-bit products, then round it once. The bound per element is therefore
    |gpu - exact| <= u |exact| + gamma_K (|A| |B|),
where u is the storage type's unit roundoff (2^-8 bf16, 2^-11 fp16), gamma_K = K 2^-24 the worst-case
float32 summation error over K terms, and |A| |B| the product of the absolute operands. A dropped or doubled
contraction chunk, a wrong tile or a transposed operand moves entries far past it.
The shapes cover:
  - the ViT-B/16 block at full size, in the launch configuration the benchmark times (256 x 256 tiles; the
    backward's two products split their contraction 3 and 9 ways);
  - 256 x 256 tiles with ragged edges, with and without a split (a 4-way split whose last part ends mid-step);
  - ragged token counts and contraction tails (D not a multiple of 64, B N not a multiple of 64);
  - the smallest legal shape;
  - a 256 x 256-tile product with one contraction step (dw with 40 tokens);
  - the small-product kernels (64 x 64 tiles with the contraction split over the 4 waves);
  - more than 4 million input features (leading dimensions past 2^22 elements).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from attn_inputs import make_case, make_proj_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, rel_l2, to_f64
from oracle import masked_attention_bwd, masked_attention_fwd, qkv_projection, qkv_projection_bwd, split_qkv

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _up(c, name):
    import torch
    a = np.ascontiguousarray(c.raw[name])
    t = torch.from_numpy(a.view(np.int16))
    return (t.view(torch.bfloat16) if c.dtype == "bf16" else t.view(torch.float16)).cuda()


def _bound(exact, absprod, K, dtype):
    return U[dtype] * np.abs(exact) + K * 2.0 ** -24 * absprod


def _check(name, gpu, exact, absprod, K, dtype):
    excess = np.abs(gpu - exact) - _bound(exact, absprod, K, dtype)
    worst = float(np.max(excess)) if excess.size else -1.0
    assert worst <= 0.0, f"{name}: an element exceeds the rounding bound by {worst:.3e}"


# (B, N, D, H, d): the ViT-B/16 block, ragged tails, the smallest shape, wide and narrow heads.
SHAPES = [
    (32, 196, 768, 12, 64),
    (2, 37, 64, 1, 32),
    (3, 50, 200, 2, 96),
    (1, 1, 8, 1, 8),
    (1, 300, 1024, 4, 128),
    (5, 7, 136, 3, 64),
    (3, 150, 520, 4, 96),
    (8, 300, 512, 4, 64),
    (1, 40, 256, 2, 128),
]


@pytest.mark.parametrize("B,N,D,H,d", SHAPES)
def test_projection_forward_and_backward(gpu_lib, B, N, D, H, d):
    import torch
    _say(f"[proj] bf16 B={B} N={N} D={D} H={H} d={d}")
    c = make_proj_case(B, N, D, H, d, "bf16", seed=B + N + D)
    x, w, dy = _up(c, "x"), _up(c, "w"), _up(c, "dqkv")
    qkv, q, k, v = gpu_lib.qkv_proj(x, w)
    dx, dw = gpu_lib.qkv_proj_bwd(x, w, dy)
    torch.cuda.synchronize()
    X, W, DY = c.f64("x"), c.f64("w"), c.f64("dqkv")
    T = B * N
    Y = qkv_projection(X, W)
    _check("qkv", to_f64(qkv), Y, qkv_projection(np.abs(X), np.abs(W)), D, "bf16")
    # The packed slices are the [B, N, H, d] views attention reads.
    assert q.data_ptr() == qkv.data_ptr() and k.stride() == qkv[:, :, 1].stride()
    DX, DW = qkv_projection_bwd(X, W, DY)
    AX, AW = qkv_projection_bwd(np.abs(X), np.abs(W), np.abs(DY))
    _check("dx", to_f64(dx), DX, AX, 3 * H * d, "bf16")
    _check("dw", to_f64(dw), DW, AW, T, "bf16")
    assert rel_l2(to_f64(dx), DX) <= TOL_GRAD_RELL2 and rel_l2(to_f64(dw), DW) <= TOL_GRAD_RELL2


def test_projection_huge_leading_dimension(gpu_lib):
    """D = 4,194,312 input features (8 tokens, one head of width 8): rows of x more than 8 MB apart, a forward
    contraction of 16,384 steps on one workgroup, and a dW product of 32,768 row tiles, all with 64-bit copy
    addresses. x is zero outside a seeded set of at most 2048 columns (runs at the start, across element 2^22 and
    at the end), so every float32 sum has at most that many nonzero terms (adding a zero is exact) and the bound
    uses that count; dW rows of the zero columns must be exactly zero."""
    import torch
    B, N, D, H, d = 1, 8, 4194312, 1, 8
    _say(f"[proj] bf16 B={B} N={N} D={D} H={H} d={d} (global_load_lds copies)")
    c = make_proj_case(B, N, D, H, d, "bf16", seed=11)
    keep = np.zeros(D, dtype=bool)
    keep[np.random.default_rng(11).choice(D, 1792, replace=False)] = True
    keep[:64] = True
    keep[(1 << 22) - 64:(1 << 22) + 64] = True
    keep[-64:] = True
    nnz = int(keep.sum())
    assert nnz <= 2048
    c.raw["x"] = np.where(keep, c.raw["x"], np.uint16(0)).astype(np.uint16)
    x, w, dy = _up(c, "x"), _up(c, "w"), _up(c, "dqkv")
    qkv, _, _, _ = gpu_lib.qkv_proj(x, w)
    dx, dw = gpu_lib.qkv_proj_bwd(x, w, dy)
    torch.cuda.synchronize()
    X, W, DY = c.f64("x"), c.f64("w"), c.f64("dqkv")
    _check("qkv", to_f64(qkv), qkv_projection(X, W), qkv_projection(np.abs(X), np.abs(W)), nnz, "bf16")
    DX, DW = qkv_projection_bwd(X, W, DY)
    AX, AW = qkv_projection_bwd(np.abs(X), np.abs(W), np.abs(DY))
    _check("dx", to_f64(dx), DX, AX, 3 * H * d, "bf16")
    dw64 = to_f64(dw)
    _check("dw", dw64, DW, AW, B * N, "bf16")
    assert not np.any(dw64[~keep]), "dw rows of all-zero x columns must be exactly zero"


def test_projection_fp16(gpu_lib):
    import torch
    B, N, D, H, d = 4, 77, 384, 6, 64
    _say(f"[proj] f16 B={B} N={N} D={D} H={H} d={d}")
    c = make_proj_case(B, N, D, H, d, "f16", seed=9)
    x, w, dy = _up(c, "x"), _up(c, "w"), _up(c, "dqkv")
    qkv, _, _, _ = gpu_lib.qkv_proj(x, w)
    dx, dw = gpu_lib.qkv_proj_bwd(x, w, dy)
    torch.cuda.synchronize()
    X, W, DY = c.f64("x"), c.f64("w"), c.f64("dqkv")
    _check("qkv", to_f64(qkv), qkv_projection(X, W), qkv_projection(np.abs(X), np.abs(W)), D, "f16")
    DX, DW = qkv_projection_bwd(X, W, DY)
    AX, AW = qkv_projection_bwd(np.abs(X), np.abs(W), np.abs(DY))
    _check("dx", to_f64(dx), DX, AX, 3 * H * d, "f16")
    _check("dw", to_f64(dw), DW, AW, B * N, "f16")


def test_projection_is_deterministic(gpu_lib):
    """Split partial sums are added in a fixed order: repeated calls give the same bits, also when the
    workspace is reused and starts out full of garbage (every call overwrites what it reads)."""
    import torch
    c = make_proj_case(8, 196, 768, 12, 64, "bf16", seed=1)
    x, w, dy = _up(c, "x"), _up(c, "w"), _up(c, "dqkv")
    assert gpu_lib.attn_qkv_proj_bwd_workspace_bytes(8, 196, 768, 12, 64) > 0   # dw splits its contraction
    ws = gpu_lib.proj_workspace_for(x, w)
    ws.fill_(255)
    r1 = gpu_lib.qkv_proj(x, w)[0], *gpu_lib.qkv_proj_bwd(x, w, dy, workspace=ws)
    r2 = gpu_lib.qkv_proj(x, w)[0], *gpu_lib.qkv_proj_bwd(x, w, dy, workspace=ws)
    r3 = gpu_lib.qkv_proj(x, w)[0], *gpu_lib.qkv_proj_bwd(x, w, dy)
    torch.cuda.synchronize()
    for a, b, c3 in zip(r1, r2, r3):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(a.view(torch.int16), c3.view(torch.int16))


def test_projection_feeds_packed_attention(gpu_lib):
    """One ViT attention block through the library: project, attend in the packed layout, back-propagate
    through attention and the projection. Every stage rounds to bf16, so the end result is held to the
    gradient bound (relative L2 5e-2) against the fp64 chain of the oracle's projection and attention."""
    import torch
    B, N, D, H, d = 2, 196, 768, 12, 64
    _say(f"[proj] block B={B} N={N} D={D} H={H} d={d}")
    c = make_proj_case(B, N, D, H, d, "bf16", seed=4)
    g = make_case(B, H, N, d, "bf16", seed=4)          # dO of the attention output
    x, w = _up(c, "x"), _up(c, "w")
    scale = g.scale
    qkv, q, k, v = gpu_lib.qkv_proj(x, w)
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, scale, layout="qkv_packed")
    do = _up(g, "do").transpose(1, 2).contiguous()     # [B, N, H, d]
    dqkv = torch.empty_like(qkv)
    ws = torch.empty(gpu_lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    gpu_lib.attn_bwd_ex(q, k, v, o, lse, do, dqkv[:, :, 0], dqkv[:, :, 1], dqkv[:, :, 2], scale, ws,
                        layout="qkv_packed")
    dx, dw = gpu_lib.qkv_proj_bwd(x, w, dqkv)
    torch.cuda.synchronize()

    X, W, DO = c.f64("x"), c.f64("w"), g.f64("do")
    Q, K, V = split_qkv(qkv_projection(X, W))
    O, _ = masked_attention_fwd(Q, K, V, scale)
    dQ, dK, dV = masked_attention_bwd(Q, K, V, DO, scale)
    DQKV = np.stack([t.transpose(0, 2, 1, 3) for t in (dQ, dK, dV)], axis=2)   # [B, N, 3, H, d]
    DX, DW = qkv_projection_bwd(X, W, DQKV)
    o_err = float(np.max(np.abs(to_f64(o).transpose(0, 2, 1, 3) - O)))
    _say(f"[proj] block: O max-abs {o_err:.2e}, dx rel-L2 {rel_l2(to_f64(dx), DX):.2e}, "
         f"dw rel-L2 {rel_l2(to_f64(dw), DW):.2e}")
    assert o_err <= TOL_BF16_O
    assert rel_l2(to_f64(dqkv), DQKV) <= TOL_GRAD_RELL2
    assert rel_l2(to_f64(dx), DX) <= TOL_GRAD_RELL2
    assert rel_l2(to_f64(dw), DW) <= TOL_GRAD_RELL2
