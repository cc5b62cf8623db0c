"""GPU checks at the edges of the shape range: a 65,536-token head, a grid of many small heads whose size is not
a multiple of the 8 XCDs, and single-token heads.

Where the oracle cannot materialise the whole head (N = 65,536: 4.3e9 scores) the forward is checked on sampled
query rows against the oracle at their positions, and the backward through identities that hold at any size
(§1 softmax rows sum to 1): sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from attn_inputs import make_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, check_lse, max_abs, rel_l2, to_device, to_f64
from oracle import masked_attention_dq_rows, attention_bwd, attention_fwd, masked_attention_fwd

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("causal", [False, True])
def test_65536_token_head(gpu_lib, causal):
    import torch
    N = 65536
    x = make_case(1, 1, N, 64, "bf16", seed=123)
    _say(f"N={N} causal={causal}")
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.forward(q, k, v, x.scale, causal=causal)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, x.scale, causal=causal)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 32767, 65535], np.random.default_rng(7).integers(0, N, 58)]))
    Q = x.f64("q", (0, 0))[rows][None, None]
    K, V = x.f64("k", (0, 0))[None, None], x.f64("v", (0, 0))[None, None]
    ro, rl = masked_attention_fwd(Q, K, V, x.scale, causal=causal, q_index=rows)
    go, gl = to_f64(o)[0, 0][rows], to_f64(lse)[0, 0][rows]
    assert max_abs(go, ro[0, 0]) <= TOL_BF16_O
    _say(f"  O max-abs {max_abs(go, ro[0, 0]):.3e}, lse error / bound {check_lse(gl, rl[0, 0], Q[0, 0], K[0, 0], x.scale, 'bf16'):.3f}")
    # dQ of the sampled rows against the oracle (each row of dQ needs only its own query and all keys).
    DO = x.f64("do", (0, 0))[rows][None, None]
    rdq = masked_attention_dq_rows(Q, K, V, DO, x.scale, causal=causal, q_index=rows)
    e_dq = rel_l2(to_f64(dq)[0, 0][rows], rdq[0, 0])
    _say(f"  dQ of {len(rows)} sampled rows: rel-L2 {e_dq:.3e}")
    assert e_dq <= TOL_GRAD_RELL2
    # Backward identities over the whole head (fp32 sums of the bf16 gradients).
    gk, gv, gdo = (t.float().sum(dim=2)[0, 0].cpu().numpy() for t in (dk, dv, do))
    scale_k = float(dk.float().abs().sum(dim=2).max())
    _say(f"  |sum dK| {np.abs(gk).max():.3e} (sum |dK| {scale_k:.3e}); sum dV - sum dO {np.abs(gv - gdo).max():.3e}")
    # bf16 rounding of each of the 65,536 rows leaves ~sqrt(N) 2^-9 |row| in the sums (observed 5e-5 and 0.04).
    assert np.abs(gk).max() <= 1e-3 * max(scale_k, 1.0)
    assert np.abs(gv - gdo).max() <= 1e-3 * np.abs(gdo).max() + 0.1
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()


def test_many_small_heads_odd_grid(gpu_lib):
    """B=37, H=13 (481 heads, a grid that is not a multiple of the 8 XCDs), N=70: whole tensors against the oracle."""
    import torch
    x = make_case(37, 13, 70, 64, "bf16", seed=124)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.forward(q, k, v, x.scale)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, x.scale)
    torch.cuda.synchronize()
    Q, K, V, DO = x.f64("q"), x.f64("k"), x.f64("v"), x.f64("do")
    ro, rl = attention_fwd(Q, K, V, x.scale)
    assert max_abs(to_f64(o), ro) <= TOL_BF16_O
    check_lse(to_f64(lse), rl, Q, K, x.scale, "bf16")
    for got, r in zip((dq, dk, dv), attention_bwd(Q, K, V, DO, x.scale)):
        assert rel_l2(to_f64(got), r) <= TOL_GRAD_RELL2


@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_single_token_heads(gpu_lib, d):
    """N = 1: O = V exactly (one weight of 1), lse = scale <q, k>, dQ = dK = 0 and dV = dO."""
    import torch
    x = make_case(3, 5, 1, d, "bf16", seed=125 + d)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.forward(q, k, v, x.scale)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, v)
    ref = x.scale * np.einsum("bhnd,bhnd->bhn", x.f64("q"), x.f64("k"))
    # One weight of exactly 1: lse is the fp32 score (d products summed, then scaled), within 1e-5.
    assert max_abs(to_f64(lse), ref) <= 1e-5
    assert torch.equal(dv, do)
    # dP and delta are the same dot product summed in two orders: their fp32 difference (~1e-6) is all that is left.
    assert max_abs(to_f64(dq), np.zeros(q.shape)) <= 1e-4 and max_abs(to_f64(dk), np.zeros(k.shape)) <= 1e-4
