"""The allocation-free backward (attn_bwd_ex_noalloc) against attn_bwd_ex, through the C ABI.

attn_bwd_ex_noalloc is attn_bwd_ex with the library's own device workspace in
place of the caller's, for callers that cannot allocate. It runs the same
kernels, so its gradients must equal attn_bwd_ex's bit for bit. Two calls in a
row, the second on a smaller input (the shared workspace still holds the first
call's contents), and neither may allocate device memory.
"""
from __future__ import annotations

import sys

import pytest

from attn_inputs import make_case
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _grads_both_ways(gpu_lib, x, causal, kv):
    import torch
    q, k, v, do = (to_device(x, n) for n in ("q", "k", "v", "do"))
    kvt = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    o, lse = gpu_lib.forward(q, k, v, x.scale, causal=causal, kv_len=kvt)
    ref = tuple(torch.empty_like(q) for _ in range(3))
    gpu_lib.attn_bwd_ex(q, k, v, o, lse, do, *ref, x.scale, gpu_lib.workspace_for(q), causal=causal, kv_len=kvt)
    got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated()
    free0, _ = torch.cuda.mem_get_info()
    gpu_lib.attn_bwd_ex_noalloc(q, k, v, o, lse, do, *got, x.scale, causal=causal, kv_len=kvt)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    return ref, got, free0 - free1


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_backward_equals_workspace_backward(gpu_lib, dtype):
    import torch
    cases = [((2, 3, 700, 64), True, [700, 411]),     # first call: causal, key padding, d = 64
             ((1, 2, 200, 128), False, None)]          # second call: a smaller input, d = 128
    for i, ((B, H, N, d), causal, kv) in enumerate(cases):
        print(f"noalloc call {i + 1}: {dtype} B={B} H={H} N={N} d={d} causal={causal} kv_len={kv}", flush=True)
        sys.stdout.flush()
        x = make_case(B, H, N, d, dtype, seed=8800 + i)
        ref, got, used = _grads_both_ways(gpu_lib, x, causal, kv)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        if i > 0:
            assert used == 0, f"device memory fell by {used} bytes during the call"
