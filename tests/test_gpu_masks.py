"""GPU parity of the masked entry points (attn_fwd_ex / attn_bwd_ex) against the masked fp64 oracle.

Masks (a reading; the article defines unmasked attention only): key padding
(kv_len[b] valid keys per batch entry) and causal (query i sees keys j <= i).
Small and ragged shapes are compared over whole tensors, including rows with
no visible key (kv_len = 0: O = 0, lse = -inf, zero gradients); the
long-sequence shapes compare whole sampled heads or sampled query rows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from attn_inputs import make_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, check_lse, max_abs, rel_l2, to_device, to_f64
from oracle import masked_attention_bwd, masked_attention_fwd

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _kv_tensor(kv):
    import torch
    return None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")


def _run(gpu_lib, x, causal, kv, bwd=True):
    import torch
    q, k, v = (to_device(x, n) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((x.B, x.H, x.N), dtype=torch.float32, device="cuda")
    kvt = _kv_tensor(kv)
    gpu_lib.attn_fwd_ex(q, k, v, o, lse, x.scale, causal=causal, kv_len=kvt)
    out = {"o": o, "lse": lse}
    if bwd:
        do = to_device(x, "do")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        gpu_lib.attn_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, x.scale, gpu_lib.workspace_for(q), causal=causal,
                            kv_len=kvt)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: to_f64(t) for n, t in out.items()}


def _check_fwd(got_o, got_lse, ro, rl, Q, K, scale):
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(got_lse), empty), "rows with no visible key must give lse = -inf"
    assert np.all(got_o[empty] == 0)
    assert max_abs(got_o, ro) <= TOL_BF16_O
    check_lse(got_lse, rl, Q, K, scale, "bf16")


def _check_grads(got, ref, kv):
    for name, r in zip(("dq", "dk", "dv"), ref):
        g = got[name]
        e = rel_l2(g, r)
        _say(f"  {name} rel-L2 {e:.3e}")
        assert e <= TOL_GRAD_RELL2, name
    # Exact zeros where the masks make a row structurally zero: keys at or past
    # kv_len[b] (no query sees them) and every query of an entry with kv_len 0.
    if kv is not None:
        for b, n in enumerate(kv):
            assert np.all(got["dk"][b, :, n:] == 0) and np.all(got["dv"][b, :, n:] == 0)
            if n == 0:
                assert np.all(got["dq"][b] == 0)


# (B, H, N, d, causal, kv_len or None)
SMALL = [
    (1, 2, 1, 64, True, None),
    (2, 2, 7, 64, True, None),
    (3, 2, 65, 64, True, [65, 33, 1]),
    (4, 2, 196, 64, False, [196, 100, 1, 0]),
    (4, 2, 196, 64, True, [196, 97, 64, 0]),
    (2, 3, 333, 64, True, None),
    (2, 1, 1000, 64, True, [1000, 517]),
    (2, 1, 1100, 64, True, None),
    (1, 2, 1088, 64, True, None),  # the pipelined forward's tiles, then its diagonal tiles (partial last block)
    (3, 1, 1100, 64, False, [1100, 1024, 333]),
    (2, 2, 129, 128, True, None),
    (1, 2, 1088, 128, True, None),  # the pipelined forward's tiles, then its diagonal tiles (partial last block)
    (3, 1, 517, 128, True, [517, 300, 0]),
    (2, 1, 1030, 128, True, [1030, 640]),
    (2, 1, 1030, 128, False, [777, 1]),
    (2, 2, 300, 32, True, [300, 45]),
    (2, 1, 1200, 32, True, None),
    (2, 2, 250, 96, True, [250, 0]),
    (2, 1, 1100, 96, True, [1100, 801]),
]


@pytest.mark.parametrize("B,H,N,d,causal,kv", SMALL)
def test_masked_fwd_bwd_parity(gpu_lib, B, H, N, d, causal, kv):
    x = make_case(B, H, N, d, "bf16", seed=3000 + N + d + 7 * B)
    _say(f"masked fwd/bwd B={B} H={H} N={N} d={d} causal={causal} kv_len={kv}")
    got = _run(gpu_lib, x, causal, kv)
    Q, K, V, DO = x.f64("q"), x.f64("k"), x.f64("v"), x.f64("do")
    ro, rl = masked_attention_fwd(Q, K, V, x.scale, causal=causal, kv_len=kv)
    _check_fwd(got["o"], got["lse"], ro, rl, Q, K, x.scale)
    _check_grads(got, masked_attention_bwd(Q, K, V, DO, x.scale, causal=causal, kv_len=kv), kv)


def test_unmasked_extended_call_equals_attn_fwd(gpu_lib):
    """attn_fwd_ex with no mask and attn_bwd_ex with no mask give bitwise the plain entry points' results."""
    import torch
    x = make_case(2, 2, 300, 64, "bf16", seed=31)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o1, l1 = gpu_lib.forward(q, k, v, x.scale)
    g1 = gpu_lib.backward(q, k, v, o1, l1, do, x.scale)
    full = _kv_tensor([300, 300])
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    gpu_lib.attn_fwd_ex(q, k, v, o2, l2, x.scale, causal=False, kv_len=full)
    g2 = tuple(torch.empty_like(q) for _ in range(3))
    gpu_lib.attn_bwd_ex(q, k, v, o2, l2, do, *g2, x.scale, gpu_lib.workspace_for(q), kv_len=full)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_out_of_range_kv_len_is_clamped(gpu_lib):
    """kv_len values below 0 or above N act as 0 and N."""
    import torch
    x = make_case(2, 1, 150, 64, "bf16", seed=32, with_grad=False)
    got = _run(gpu_lib, x, False, [-5, 10 ** 6], bwd=False)
    ro, rl = masked_attention_fwd(x.f64("q"), x.f64("k"), x.f64("v"), x.scale, kv_len=[0, 150])
    _check_fwd(got["o"], got["lse"], ro, rl, x.f64("q"), x.f64("k"), x.scale)
    del torch


def test_masked_backward_is_deterministic(gpu_lib):
    x = make_case(2, 2, 700, 64, "bf16", seed=33)
    a = _run(gpu_lib, x, True, [700, 411])
    b = _run(gpu_lib, x, True, [700, 411])
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n], equal_nan=False), n


def _head(x, name, b, h):
    return x.f64(name, (b, h))[None, None]


@pytest.mark.parametrize("causal,kv", [(True, None), (False, [4096, 3001, 1, 2048, 4095, 17, 4000, 0]),
                                       (True, [4096, 2500, 64, 1000, 3333, 129, 4096, 1])])
def test_long_sequence_masked_sampled_heads(gpu_lib, causal, kv):
    """B=8, H=16, N=4096, d=64 (the long-sequence shape): three whole heads against the oracle."""
    x = make_case(8, 16, 4096, 64, "bf16", seed=34)
    _say(f"long masked causal={causal} kv_len={kv}")
    got = _run(gpu_lib, x, causal, kv)
    for (b, h) in ((0, 0), (1, 7), (5, 15)):
        Q, K, V, DO = (_head(x, n, b, h) for n in ("q", "k", "v", "do"))
        kvb = None if kv is None else [kv[b]]
        ro, rl = masked_attention_fwd(Q, K, V, x.scale, causal=causal, kv_len=kvb)
        _check_fwd(got["o"][b:b + 1, h:h + 1], got["lse"][b:b + 1, h:h + 1], ro, rl, Q, K, x.scale)
        ref = masked_attention_bwd(Q, K, V, DO, x.scale, causal=causal, kv_len=kvb)
        _check_grads({n: got[n][b:b + 1, h:h + 1] for n in ("dq", "dk", "dv")}, ref, kvb)
    if kv is not None and 0 in kv:
        b0 = kv.index(0)
        assert np.all(got["o"][b0] == 0) and np.all(np.isneginf(got["lse"][b0]))
        assert np.all(got["dq"][b0] == 0) and np.all(got["dk"][b0] == 0) and np.all(got["dv"][b0] == 0)


def test_very_long_causal_forward_sampled_rows(gpu_lib):
    """B=2, H=16, N=16384, d=128, causal: 96 query rows of two heads against the oracle at their positions."""
    x = make_case(2, 16, 16384, 128, "bf16", seed=35, with_grad=False)
    got = _run(gpu_lib, x, True, None, bwd=False)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 255, 256, 8191, 16383],
                                     np.random.default_rng(35).integers(0, 16384, 86)]))
    for (b, h) in ((0, 3), (1, 14)):
        Q = x.f64("q", (b, h))[rows][None, None]
        K, V = _head(x, "k", b, h), _head(x, "v", b, h)
        ro, rl = masked_attention_fwd(Q, K, V, x.scale, causal=True, q_index=rows)
        _check_fwd(got["o"][b, h][rows][None, None], got["lse"][b, h][rows][None, None], ro, rl, Q, K, x.scale)
