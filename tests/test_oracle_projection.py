"""Pins for the query/key/value projection oracle (oracle/projection.py).

Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention" (German edition
of the self-attention / Triton / FlashAttention article, itimpress.au,
2026-11-15), §1 first bullet: Q = X W_Q, K = X W_K, V = X W_V, one set of
weights per head. No GPU is involved. Each pin targets a plausible slip:
  - X^T in place of X, or W^T in place of W: hand example, brute force;
  - Q, K, V or the heads swapped in the packed output: identity weights;
  - a transposed or unsummed weight gradient: finite differences, adjoint
    identity;
  - the wrong axis order when the packed output is split into per-head
    arrays: identity weights through split_qkv.
"""
import json
import os

import numpy as np
import pytest

from attn_inputs import make_proj_case
from oracle import attention_fwd, brute_qkv_projection, qkv_projection, qkv_projection_bwd, split_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_proj.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_derived_example(case):
    """tests/golden/hand_proj.json, derived by hand from §1's three products."""
    x, w, dy = (np.array(case[n]) for n in ("x", "w", "dqkv"))
    np.testing.assert_array_equal(qkv_projection(x, w), np.array(case["qkv"]))
    dx, dw = qkv_projection_bwd(x, w, dy)
    np.testing.assert_array_equal(dx, np.array(case["dx"]))
    np.testing.assert_array_equal(dw, np.array(case["dw"]))


@pytest.mark.parametrize("B,N,D,H,d", [(1, 1, 1, 1, 1), (1, 3, 2, 1, 2), (2, 3, 5, 2, 3), (2, 4, 3, 3, 1)])
def test_brute_force(B, N, D, H, d):
    """Single dot products with math.fsum agree with the oracle to 1e-12."""
    rng = np.random.default_rng(B * 1000 + N * 100 + D * 10 + H + d)
    x = rng.standard_normal((B, N, D))
    w = rng.standard_normal((D, 3, H, d))
    np.testing.assert_allclose(qkv_projection(x, w), brute_qkv_projection(x, w), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,N,H,d", [(1, 2, 1, 4), (2, 3, 2, 3), (2, 5, 3, 2)])
def test_identity_weights_select_features(B, N, H, d):
    """With D = 3 H d and w = identity, qkv[b, n, t, h, j] = x[b, n, (t H + h) d + j] exactly,
    and split_qkv returns Q, K, V of head h as columns (t H + h) d .. + d of X."""
    D = 3 * H * d
    rng = np.random.default_rng(11 * B + N + H + d)
    x = rng.standard_normal((B, N, D))
    w = np.eye(D).reshape(D, 3, H, d)
    qkv = qkv_projection(x, w)
    for t in range(3):
        for h in range(H):
            c0 = (t * H + h) * d
            np.testing.assert_array_equal(qkv[:, :, t, h, :], x[:, :, c0:c0 + d])
    q, k, v = split_qkv(qkv)
    for t, a in enumerate((q, k, v)):
        assert a.shape == (B, H, N, d)
        for h in range(H):
            c0 = (t * H + h) * d
            np.testing.assert_array_equal(a[:, h], x[:, :, c0:c0 + d])


@pytest.mark.parametrize("B,N,D,H,d", [(1, 2, 3, 1, 2), (2, 3, 4, 2, 1)])
def test_gradients_match_finite_differences(B, N, D, H, d):
    """Analytic dx, dw equal central differences of sum(qkv * dqkv)."""
    rng = np.random.default_rng(3 + B + N + D + H + d)
    x = rng.standard_normal((B, N, D))
    w = rng.standard_normal((D, 3, H, d))
    dy = rng.standard_normal((B, N, 3, H, d))
    dx, dw = qkv_projection_bwd(x, w, dy)
    h = 1e-6

    def loss(xx, ww):
        return float(np.sum(brute_qkv_projection(xx, ww) * dy))

    for arr, grad, which in ((x, dx, 0), (w, dw, 1)):
        fd = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            lp = loss(p, w) if which == 0 else loss(x, p)
            lm = loss(m, w) if which == 0 else loss(x, m)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7)


def test_adjoint_identity():
    """<P(x, w), dy> = <x, dx> = <w, dw>: the gradients are the adjoints of the
    linear map in x and in w (holds for any shapes; checked on a mid-sized case)."""
    c = make_proj_case(3, 17, 48, 2, 16, "bf16", seed=5)
    x, w, dy = c.f64("x"), c.f64("w"), c.f64("dqkv")
    y = qkv_projection(x, w)
    dx, dw = qkv_projection_bwd(x, w, dy)
    a = float(np.sum(y * dy))
    assert abs(float(np.sum(x * dx)) - a) <= 1e-10 * (1 + abs(a))
    assert abs(float(np.sum(w * dw)) - a) <= 1e-10 * (1 + abs(a))


def test_projection_feeds_attention_per_head():
    """Attention of head h on split_qkv's output equals attention on that head's own
    products X W_Q[h], X W_K[h], X W_V[h], formed one head at a time."""
    c = make_proj_case(2, 9, 24, 3, 8, "bf16", seed=2)
    x, w = c.f64("x"), c.f64("w")
    q, k, v = split_qkv(qkv_projection(x, w))
    scale = 8 ** -0.5
    for b in range(2):
        for h in range(3):
            qh, kh, vh = (x[b] @ w[:, t, h, :] for t in range(3))
            o_ref, l_ref = attention_fwd(qh, kh, vh, scale)
            o, l = attention_fwd(q[b, h], k[b, h], v[b, h], scale)
            np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(l, l_ref, rtol=1e-12, atol=1e-12)


def test_generator_weight_spread():
    """w ~ N(0, 1/D): projected values come out near unit spread."""
    c = make_proj_case(4, 64, 256, 2, 32, "bf16", seed=0)
    y = qkv_projection(c.f64("x"), c.f64("w"))
    assert 0.9 < float(np.std(y)) < 1.1
