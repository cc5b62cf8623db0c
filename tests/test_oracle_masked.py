"""Pins for the masked oracle (key padding and causal masks), CPU only.

The article ("Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention", §1
"Attention" formula) defines unmasked attention; the masks are the reading
documented in oracle/masked.py. Each pin ties the masked definition to
something computed another way: the unmasked oracle on truncated keys, a
pure-Python brute force that skips masked pairs, finite differences, closed
forms and torch's CPU fp64 routine. A mask off by one (j < i instead of
j <= i), a transposed mask or a padding length off by one fails several.
"""
import math

import numpy as np
import pytest

from oracle import (attention_bwd, attention_fwd, brute_attention_fwd, brute_attention_grads_fd,
                    masked_attention_bwd, masked_attention_dq_rows, masked_attention_ds, masked_attention_fwd,
                    visible_keys)


def _r(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def test_visible_keys_pattern():
    vis = visible_keys(5, np.arange(5), True, 3)
    expect = np.array([[1, 0, 0, 0, 0], [1, 1, 0, 0, 0], [1, 1, 1, 0, 0], [1, 1, 1, 0, 0], [1, 1, 1, 0, 0]], bool)
    np.testing.assert_array_equal(vis, expect)
    np.testing.assert_array_equal(visible_keys(4, np.arange(2), False, 2), [[1, 1, 0, 0], [1, 1, 0, 0]])


@pytest.mark.parametrize("causal,kv", [(True, None), (False, [3]), (True, [4]), (True, [0])])
def test_brute_force_masked_forward(causal, kv):
    """Pure-Python loops that skip masked pairs agree with the vectorised masked oracle to 1e-12."""
    rng = np.random.default_rng(40)
    N, d = 6, 3
    q, k, v = _r(rng, 1, 1, N, d), _r(rng, 1, 1, N, d), _r(rng, 1, 1, N, 2)
    vis = visible_keys(N, np.arange(N), causal, N if kv is None else kv[0])
    ob, lb = brute_attention_fwd(q[0, 0], k[0, 0], v[0, 0], 0.7, vis.tolist())
    o, lse = masked_attention_fwd(q, k, v, 0.7, causal=causal, kv_len=kv)
    np.testing.assert_allclose(o[0, 0], np.array(ob), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse[0, 0]), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[0, 0][fin], np.array(lb)[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal,kv", [(True, None), (False, [2]), (True, [3])])
def test_masked_gradients_match_finite_differences(causal, kv):
    rng = np.random.default_rng(41)
    N, d = 4, 2
    q, k, v, do = (_r(rng, 1, 1, N, d) for _ in range(4))
    vis = visible_keys(N, np.arange(N), causal, N if kv is None else kv[0])
    fq, fk, fv = brute_attention_grads_fd(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.6, allowed=vis.tolist())
    dq, dk, dv = masked_attention_bwd(q, k, v, do, 0.6, causal=causal, kv_len=kv)
    for a, f in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a[0, 0], f, rtol=1e-6, atol=1e-8)


def test_causal_row_equals_unmasked_attention_over_its_prefix():
    """Causal row i is the unmasked definition over keys 0..i (a different code path)."""
    rng = np.random.default_rng(42)
    B, H, N, d = 2, 2, 37, 8
    q, k, v = _r(rng, B, H, N, d), _r(rng, B, H, N, d), _r(rng, B, H, N, 5)
    o, lse = masked_attention_fwd(q, k, v, 0.3, causal=True)
    for i in (0, 1, 2, 17, 36):
        o1, l1 = attention_fwd(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.3)
        np.testing.assert_allclose(o[:, :, i:i + 1], o1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i:i + 1], l1, rtol=0, atol=1e-13)
    # Row 0 sees only key 0: O_0 = v_0 and lse_0 = s_00 exactly.
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), rtol=1e-15)


def test_key_padding_equals_truncated_keys_forward_and_backward():
    """kv_len[b] keys: same as the unmasked oracle on K[:len], V[:len]; dK, dV of padded keys are 0."""
    rng = np.random.default_rng(43)
    B, H, N, d = 3, 2, 21, 6
    q, k, v, do = _r(rng, B, H, N, d), _r(rng, B, H, N, d), _r(rng, B, H, N, d), _r(rng, B, H, N, d)
    kv = [21, 8, 1]
    o, lse = masked_attention_fwd(q, k, v, 0.45, kv_len=kv)
    dq, dk, dv = masked_attention_bwd(q, k, v, do, 0.45, kv_len=kv)
    for b, n in enumerate(kv):
        o1, l1 = attention_fwd(q[b], k[b, :, :n], v[b, :, :n], 0.45)
        np.testing.assert_allclose(o[b], o1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], l1, rtol=0, atol=1e-13)
        g = attention_bwd(q[b], k[b, :, :n], v[b, :, :n], do[b], 0.45)
        np.testing.assert_allclose(dq[b], g[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk[b, :, :n], g[1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[b, :, :n], g[2], rtol=0, atol=1e-13)
        assert np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0)


def test_causal_identical_keys_closed_form():
    """All keys equal under the causal mask: O_i = mean(v_0..v_i), lse_i = s_i + ln(i + 1)."""
    rng = np.random.default_rng(44)
    N, d = 19, 4
    q = _r(rng, 1, 1, N, d)
    k = np.tile(_r(rng, 1, 1, 1, d), (1, 1, N, 1))
    v = _r(rng, 1, 1, N, 3)
    o, lse = masked_attention_fwd(q, k, v, 0.5, causal=True)
    means = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], means, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], 0.5 * (q[0, 0] @ k[0, 0, 0]) + np.log(np.arange(1, N + 1)), atol=1e-13)


def test_rows_without_keys():
    """kv_len = 0: every row is empty, O = 0, lse = -inf, and no gradient flows."""
    rng = np.random.default_rng(45)
    q, k, v, do = (_r(rng, 2, 1, 5, 4) for _ in range(4))
    o, lse = masked_attention_fwd(q, k, v, 0.5, causal=True, kv_len=[0, 5])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))
    dq, dk, dv = masked_attention_bwd(q, k, v, do, 0.5, causal=True, kv_len=[0, 5])
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)


def test_causal_backward_invariants():
    """Every causal row has a visible key: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i still hold."""
    rng = np.random.default_rng(46)
    q, k, v, do = (_r(rng, 1, 2, 23, 5) for _ in range(4))
    dq, dk, dv = masked_attention_bwd(q, k, v, do, 0.4, causal=True)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # The first key is seen by every row, the last by one row only: dV_{N-1} = P_{N-1,N-1} dO_{N-1}.
    o, lse = masked_attention_fwd(q, k, v, 0.4, causal=True)
    p_last = np.exp(0.4 * np.einsum("bhd,bhd->bh", q[:, :, -1], k[:, :, -1]) - lse[:, :, -1])
    np.testing.assert_allclose(dv[:, :, -1], p_last[..., None] * do[:, :, -1], atol=1e-13)


def test_sampled_rows_match_full_rows():
    """q_index places a few rows at their sequence positions (used for long-sequence checks)."""
    rng = np.random.default_rng(47)
    q, k, v = _r(rng, 2, 1, 40, 4), _r(rng, 2, 1, 40, 4), _r(rng, 2, 1, 40, 4)
    o, lse = masked_attention_fwd(q, k, v, 0.5, causal=True, kv_len=[30, 40])
    rows = np.array([0, 3, 29, 31, 39])
    o2, lse2 = masked_attention_fwd(q[:, :, rows], k, v, 0.5, causal=True, kv_len=[30, 40], q_index=rows)
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(lse2, lse[:, :, rows])


@pytest.mark.parametrize("causal,kv", [(True, None), (False, [25, 40]), (True, [30, 7])])
def test_dq_rows_match_full_backward(causal, kv):
    """dQ of sampled rows at their sequence positions equals those rows of the full masked backward (itself pinned
    by finite differences), including rows with no visible key (dQ = 0)."""
    rng = np.random.default_rng(48)
    q, k, v, do = (_r(rng, 2, 2, 40, 4) for _ in range(4))
    dq = masked_attention_bwd(q, k, v, do, 0.45, causal=causal, kv_len=kv)[0]
    rows = np.array([0, 1, 6, 7, 24, 25, 39])
    got = masked_attention_dq_rows(q[:, :, rows], k, v, do[:, :, rows], 0.45, causal=causal, kv_len=kv,
                                   q_index=rows)
    np.testing.assert_allclose(got, dq[:, :, rows], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal,kv", [(True, None), (False, [2]), (True, [3])])
def test_masked_score_gradient_from_finite_differences(causal, kv):
    """dS against finite differences: with N = d keys and an invertible K, dQ = scale dS K fixes
    dS = dQ_fd K^-1 / scale from brute-force differences alone; 0 on masked pairs."""
    rng = np.random.default_rng(50)
    N = d = 3
    q, k, v, do = (_r(rng, 1, 1, N, d) for _ in range(4))
    vis = visible_keys(N, np.arange(N), causal, N if kv is None else kv[0])
    fq, _, _ = brute_attention_grads_fd(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.6, allowed=vis.tolist())
    ds = masked_attention_ds(q, k, v, do, 0.6, causal=causal, kv_len=kv)[0, 0]
    np.testing.assert_allclose(ds, fq @ np.linalg.inv(k[0, 0]) / 0.6, rtol=1e-5, atol=1e-8)
    assert np.all(ds[~vis] == 0)


def test_dq_rows_match_finite_differences():
    """The per-row dQ against central differences of sum(O * dO) over the given rows (causal, tiny case)."""
    rng = np.random.default_rng(49)
    N, d, rows = 6, 3, np.array([1, 4])
    q, k, v, do = (_r(rng, 1, 1, N, d) for _ in range(4))
    got = masked_attention_dq_rows(q[:, :, rows], k, v, do[:, :, rows], 0.8, causal=True, q_index=rows)
    h = 1e-6
    for r, i in enumerate(rows):
        for c in range(d):
            qp, qm = q.copy(), q.copy()
            qp[0, 0, i, c] += h
            qm[0, 0, i, c] -= h
            fp = (masked_attention_fwd(qp, k, v, 0.8, causal=True)[0][0, 0, rows] * do[0, 0, rows]).sum()
            fm = (masked_attention_fwd(qm, k, v, 0.8, causal=True)[0][0, 0, rows] * do[0, 0, rows]).sum()
            assert abs(got[0, 0, r, c] - (fp - fm) / (2 * h)) <= 1e-7


def test_torch_cpu_fp64_masked_cross_check():
    """torch CPU fp64 scaled_dot_product_attention with a boolean mask + autograd agrees."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(48)
    B, H, N, d = 2, 2, 13, 8
    q, k, v, do = (_r(rng, B, H, N, d) for _ in range(4))
    kv = [13, 6]
    allowed = np.stack([visible_keys(N, np.arange(N), True, n) for n in kv])[:, None]
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(allowed), scale=0.35)
    to.backward(torch.tensor(do))
    o, _ = masked_attention_fwd(q, k, v, 0.35, causal=True, kv_len=kv)
    dq, dk, dv = masked_attention_bwd(q, k, v, do, 0.35, causal=True, kv_len=kv)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-13)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_unmasked_reading_is_the_plain_oracle():
    """causal=False and kv_len=None reduce to the unmasked definition exactly."""
    rng = np.random.default_rng(49)
    q, k, v, do = (_r(rng, 2, 3, 11, 4) for _ in range(4))
    o, lse = masked_attention_fwd(q, k, v, 0.7)
    o1, l1 = attention_fwd(q, k, v, 0.7)
    np.testing.assert_allclose(o, o1, atol=1e-14)
    np.testing.assert_allclose(lse, l1, atol=1e-14)
    for a, b in zip(masked_attention_bwd(q, k, v, do, 0.7), attention_bwd(q, k, v, do, 0.7)):
        np.testing.assert_allclose(a, b, atol=1e-13)
    assert math.isfinite(float(lse.min()))
