"""Pins for the fp64 CPU oracle, against what the article and mathematics fix.

Article: "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention" (German edition
of the self-attention / Triton / FlashAttention article, itimpress.au,
2026-11-15), §1 ("Scores" and "Attention" formulas, row-wise softmax whose rows
sum to 1, independent heads) and §3 (backward rebuilt from saved row
statistics). No GPU is involved; each pin is chosen so that a plausible slip
in the oracle (a dropped scale, a transposed product, a softmax over the wrong
axis, a log in the wrong base, a sign error in a gradient) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_bwd, attention_ds, attention_fwd, attention_probs, brute_attention_fwd,
                    brute_attention_grads_fd)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_2x2.json")


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_derived_examples(case):
    """Hand-derived 2x2 examples (tests/golden/hand_2x2.json, derived from §1's formulas)."""
    q, k, v, do = (np.array(case[n]) for n in ("q", "k", "v", "do"))
    o, lse = attention_fwd(q, k, v, case["scale"])
    np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, case["lse"], rtol=0, atol=1e-14)
    dq, dk, dv = attention_bwd(q, k, v, do, case["scale"])
    np.testing.assert_allclose(dq, case["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, case["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, case["dv"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("M,N,d,dv", [(1, 1, 1, 1), (2, 3, 2, 2), (5, 4, 3, 2), (8, 8, 4, 3), (3, 7, 2, 5)])
def test_brute_force_forward(M, N, d, dv):
    """Pure-Python loops (no max shift, fsum) agree with the oracle to 1e-12 on tiny inputs."""
    rng = np.random.default_rng(M * 100 + N * 10 + d)
    q, k, v = _rand(rng, M, d), _rand(rng, N, d), _rand(rng, N, dv)
    scale = 0.7
    o_b, lse_b = brute_attention_fwd(q, k, v, scale)
    o, lse = attention_fwd(q, k, v, scale)
    np.testing.assert_allclose(o, np.array(o_b), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lse_b), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,N,d", [(2, 2, 2), (3, 5, 2), (4, 3, 3)])
def test_gradients_match_finite_differences(M, N, d):
    """Analytic backward equals central finite differences of sum(O * dO) through the brute forward."""
    rng = np.random.default_rng(7 + M + N + d)
    q, k, v, do = _rand(rng, M, d), _rand(rng, N, d), _rand(rng, N, d), _rand(rng, M, d)
    scale = 0.6
    dq, dk, dv = attention_bwd(q, k, v, do, scale)
    fq, fk, fv = brute_attention_grads_fd(q, k, v, do, scale)
    for a, f in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, f, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("N", [2, 3])
def test_score_gradient_from_finite_differences(N):
    """dS (the gradient with respect to the scaled scores) against finite differences: with N = d keys and an
    invertible K, dQ = scale dS K fixes dS = dQ_fd K^-1 / scale from the brute-force differences alone. Its rows
    sum to 0 (the softmax ignores a common shift of a row)."""
    rng = np.random.default_rng(70 + N)
    M, d, scale = 3, N, 0.7
    q, k, v, do = _rand(rng, M, d), _rand(rng, N, d), _rand(rng, N, 2), _rand(rng, M, 2)
    fq, _, _ = brute_attention_grads_fd(q, k, v, do, scale)
    ds = attention_ds(q, k, v, do, scale)
    np.testing.assert_allclose(ds, fq @ np.linalg.inv(k) / scale, rtol=1e-5, atol=1e-8)
    np.testing.assert_allclose(ds.sum(axis=1), 0.0, atol=1e-14)


def test_torch_cpu_fp64_cross_check():
    """The textbook library routine (torch CPU fp64 SDPA + autograd) agrees on a few small heads."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    B, H, M, N, d = 2, 3, 9, 11, 8
    q, k, v, do = _rand(rng, B, H, M, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, M, d)
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    to.backward(torch.tensor(do, dtype=torch.float64))
    o, _ = attention_fwd(q, k, v, scale)
    dq, dk, dv = attention_bwd(q, k, v, do, scale)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- invariants and closed forms

def test_rows_sum_to_one():
    """§1 softmax paragraph: each probability row sums to 1 (and softmax runs over keys, not queries)."""
    rng = np.random.default_rng(11)
    q, k = _rand(rng, 2, 3, 17, 8, scale=3.0), _rand(rng, 2, 3, 29, 8, scale=3.0)
    p = attention_probs(q, k, 0.35)
    assert p.shape == (2, 3, 17, 29)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    # The column sums are not 1 in general: a softmax over the wrong axis fails this.
    assert np.max(np.abs(p.sum(axis=-2) - 1.0)) > 1e-3


def test_identical_keys_give_mean_of_values():
    """All keys equal => uniform weights: O_i = mean_j v_j and lse_i = s_i + ln N."""
    rng = np.random.default_rng(12)
    N, d = 13, 6
    q = _rand(rng, 5, d)
    k = np.tile(_rand(rng, 1, d), (N, 1))
    v = _rand(rng, N, d)
    scale = 0.4
    o, lse = attention_fwd(q, k, v, scale)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (5, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, scale * (q @ k[0]) + math.log(N), rtol=0, atol=1e-12)


def test_zero_scale_gives_mean_and_log_n():
    """scale = 0 => every score is 0: O = mean(V), lse = ln N (natural log)."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 7, 4), _rand(rng, 196, 4), _rand(rng, 196, 4)
    o, lse = attention_fwd(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (7, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(196), rtol=0, atol=1e-13)


def test_one_dominant_score_returns_that_value_row():
    """A score that beats the rest of its row by margin >= 20 returns that V row, within (N-1) e^-20 max|v|."""
    rng = np.random.default_rng(14)
    N, d = 64, 16
    q, k, v = _rand(rng, 4, d), _rand(rng, N, d), _rand(rng, N, d)
    scale = 1.0
    picks = [5, 17, 33, 60]
    for i, j in enumerate(picks):
        k[j] = q[i] * 40.0 / np.dot(q[i], q[i])     # score(i, j) = 40
    s = (q @ k.T) * scale
    for i, j in enumerate(picks):
        other = np.delete(s[i], j)
        assert s[i, j] - other.max() >= 20
    o, _ = attention_fwd(q, k, v, scale)
    bound = (N - 1) * math.exp(-20) * np.abs(v).max() * 2
    for i, j in enumerate(picks):
        np.testing.assert_allclose(o[i], v[j], rtol=0, atol=bound)


def test_permutation_invariance():
    """Permuting K and V rows together leaves O unchanged; permuting Q rows permutes O's rows."""
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 11, 5), _rand(rng, 23, 5), _rand(rng, 23, 7)
    o, lse = attention_fwd(q, k, v, 0.8)
    perm = rng.permutation(23)
    o2, lse2 = attention_fwd(q, k[perm], v[perm], 0.8)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    # Permuting K alone changes the result (guards against a kernel that ignores the pairing).
    o3, _ = attention_fwd(q, k[perm], v, 0.8)
    assert np.max(np.abs(o3 - o)) > 1e-3
    qperm = rng.permutation(11)
    o4, lse4 = attention_fwd(q[qperm], k, v, 0.8)
    np.testing.assert_allclose(o4, o[qperm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse4, lse[qperm], rtol=0, atol=1e-13)


def test_key_shift_invariance():
    """Adding u to every key leaves O unchanged and shifts lse_i by scale * <q_i, u>."""
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 9, 6), _rand(rng, 31, 6), _rand(rng, 31, 6)
    u = _rand(rng, 6, scale=5.0)
    o, lse = attention_fwd(q, k, v, 0.5)
    o2, lse2 = attention_fwd(q, k + u, v, 0.5)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 0.5 * (q @ u), rtol=0, atol=1e-11)


def test_value_affinity():
    """V -> a V + 1 b^T gives O -> a O + 1 b^T (rows of P sum to 1)."""
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 6, 4), _rand(rng, 10, 4), _rand(rng, 10, 3)
    b = _rand(rng, 3)
    o, _ = attention_fwd(q, k, v, 1.1)
    o2, _ = attention_fwd(q, k, -2.5 * v + b, 1.1)
    np.testing.assert_allclose(o2, -2.5 * o + b, rtol=0, atol=1e-12)


def test_heads_are_independent():
    """§1 last paragraph: each (batch, head) slice equals a single-head call on that slice."""
    rng = np.random.default_rng(18)
    q, k, v, do = (_rand(rng, 2, 3, 12, 4) for _ in range(4))
    o, lse = attention_fwd(q, k, v, 0.5)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5)
    for b in range(2):
        for h in range(3):
            o1, lse1 = attention_fwd(q[b, h], k[b, h], v[b, h], 0.5)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], lse1)
            g = attention_bwd(q[b, h], k[b, h], v[b, h], do[b, h], 0.5)
            for full, one in zip((dq, dk, dv), g):
                np.testing.assert_array_equal(full[b, h], one)


def test_large_scores_stay_finite():
    """Scores beyond exp's fp64 range (|s| > 709) still give finite results equal to the unshifted problem."""
    rng = np.random.default_rng(19)
    q, k, v = _rand(rng, 8, 64, scale=8.0), _rand(rng, 50, 64, scale=8.0), _rand(rng, 50, 64)
    o, lse = attention_fwd(q, k, v, 0.125)
    u = q[0] * (8000.0 / np.dot(q[0], q[0]))          # shifts row 0's scores by +1000
    o2, lse2 = attention_fwd(q, k + u, v, 0.125)
    assert np.max(np.abs((q @ (k + u).T) * 0.125)) > 900
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(lse2))
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse2, lse + 0.125 * (q @ u), rtol=1e-12, atol=1e-9)


# ---------------------------------------------------------------- backward invariants

def test_backward_invariants():
    """sum_j dS_ij = 0 => sum_j dK_j = 0; sum_j dV_j = sum_i dO_i; D_i = <dO_i, O_i> = sum_j P_ij dP_ij."""
    rng = np.random.default_rng(20)
    q, k, v, do = _rand(rng, 14, 5), _rand(rng, 19, 5), _rand(rng, 19, 5), _rand(rng, 14, 5)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.45)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)
    o, _ = attention_fwd(q, k, v, 0.45)
    p = attention_probs(q, k, 0.45)
    np.testing.assert_allclose((do * o).sum(axis=1), (p * (do @ v.T)).sum(axis=1), rtol=1e-12, atol=1e-13)


def test_equal_value_rows_zero_qk_gradients():
    """All V rows equal => O does not depend on Q or K: dQ = dK = 0, while dV = P^T dO."""
    rng = np.random.default_rng(21)
    q, k, do = _rand(rng, 9, 4), _rand(rng, 12, 4), _rand(rng, 9, 3)
    v = np.tile(_rand(rng, 1, 3), (12, 1))
    dq, dk, dv = attention_bwd(q, k, v, do, 0.9)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, attention_probs(q, k, 0.9).T @ do, rtol=1e-13, atol=1e-13)


def test_rectangular_and_batched_shapes():
    """Oracle accepts M != N and leading batch dims; O has q's rows and v's width."""
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 2, 5, 3), _rand(rng, 2, 8, 3), _rand(rng, 2, 8, 6)
    o, lse = attention_fwd(q, k, v, 1.0)
    assert o.shape == (2, 5, 6) and lse.shape == (2, 5)
    with pytest.raises(ValueError):
        attention_fwd(q, k[:, :7], v, 1.0)
