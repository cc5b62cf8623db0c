"""GPU parity of the fp16 path (attn_fwd_ex / attn_bwd_ex with ATTN_DTYPE_F16) against the fp64 oracle.

fp16 storage is a reading of the article's unmasked definition (§1
"Attention" formula) in another 16-bit type: inputs are rounded to IEEE
binary16 by the generator, the oracle runs on those exact values, and the
kernels use the fp16 matrix-core product with fp32 accumulation.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from attn_inputs import make_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, check_lse, max_abs, rel_l2, to_device, to_f64
from oracle import attention_bwd, attention_fwd, masked_attention_bwd, masked_attention_fwd

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _kv(kv):
    import torch
    return None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("B,H,N,d,causal,kv", [
    (1, 1, 1, 64, False, None), (2, 3, 65, 64, False, None), (2, 2, 196, 64, False, None),
    (2, 2, 333, 64, True, [333, 120]), (1, 2, 1100, 64, False, None), (2, 1, 1100, 64, True, None),
    (1, 2, 129, 128, False, None), (2, 1, 517, 128, True, [517, 0]), (1, 1, 1030, 128, False, [700]),
    (2, 2, 200, 32, True, None), (1, 1, 1050, 96, False, None),
    (1, 2, 1100, 128, False, None),  # the ping-pong forward (unmasked, N >= 1024, d = 128), ragged last tile
])
def test_f16_fwd_bwd_parity(gpu_lib, B, H, N, d, causal, kv):
    import torch
    x = make_case(B, H, N, d, "f16", seed=5000 + N + d)
    _say(f"f16 fwd/bwd B={B} H={H} N={N} d={d} causal={causal} kv_len={kv}")
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    assert q.dtype == torch.float16
    o, lse = gpu_lib.forward(q, k, v, x.scale, causal=causal, kv_len=_kv(kv))
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, x.scale, causal=causal, kv_len=_kv(kv))
    torch.cuda.synchronize()
    Q, K, V, DO = x.f64("q"), x.f64("k"), x.f64("v"), x.f64("do")
    ro, rl = masked_attention_fwd(Q, K, V, x.scale, causal=causal, kv_len=kv)
    go, gl = to_f64(o), to_f64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty) and np.all(go[empty] == 0)
    e_o = max_abs(go, ro)
    _say(f"  O max-abs {e_o:.3e}")
    assert e_o <= TOL_BF16_O
    _say(f"  lse error / bound {check_lse(gl, rl, Q, K, x.scale, 'f16'):.3f}")
    ref = masked_attention_bwd(Q, K, V, DO, x.scale, causal=causal, kv_len=kv)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = rel_l2(to_f64(got), r)
        _say(f"  {name} rel-L2 {e:.3e}")
        assert e <= TOL_GRAD_RELL2, name


def test_f16_is_more_accurate_than_bf16(gpu_lib):
    """Same values in both 16-bit types (exactly representable in each): fp16 rounds P and O finer."""
    import torch
    x = make_case(2, 2, 300, 64, "bf16", seed=41)
    Q, K, V = x.f64("q"), x.f64("k"), x.f64("v")
    for a in (Q, K, V):  # below fp16's normal range a bf16 value may not be exact in fp16
        a[np.abs(a) < 2.0 ** -12] = 0.0
    ro, _ = attention_fwd(Q, K, V, x.scale)
    errs = {}
    for dt in (torch.bfloat16, torch.float16):
        # bf16 values in fp16's normal range are exact in fp16 as well (8 <= 11 significant bits).
        q, k, v = (torch.from_numpy(a).to(dt).cuda() for a in (Q, K, V))
        assert torch.equal(q.double().cpu(), torch.from_numpy(Q))
        o, _ = gpu_lib.forward(q, k, v, x.scale)
        torch.cuda.synchronize()
        errs[dt] = max_abs(to_f64(o), ro)
    _say(f"O max-abs bf16 {errs[torch.bfloat16]:.2e} fp16 {errs[torch.float16]:.2e}")
    assert errs[torch.float16] < errs[torch.bfloat16] / 4


def test_f16_long_sequence_sampled_heads(gpu_lib):
    """B=8, H=16, N=4096, d=64 in fp16: two whole heads of forward and backward against the oracle."""
    import torch
    x = make_case(8, 16, 4096, 64, "f16", seed=42)
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.forward(q, k, v, x.scale)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, x.scale)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (6, 11)):
        Q, K, V, DO = (x.f64(n, (b, h)) for n in ("q", "k", "v", "do"))
        ro, rl = attention_fwd(Q, K, V, x.scale)
        assert max_abs(to_f64(o[b, h]), ro) <= TOL_BF16_O
        check_lse(to_f64(lse[b, h]), rl, Q, K, x.scale, "f16")
        for got, r in zip((dq, dk, dv), attention_bwd(Q, K, V, DO, x.scale)):
            assert rel_l2(to_f64(got[b, h]), r) <= TOL_GRAD_RELL2
