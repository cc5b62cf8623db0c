"""GPU pins of the online softmax and of the backward's closed forms.

Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention", §3, online-softmax
bullet: a running row maximum and normaliser rescale the partial output as the
key tiles arrive, so the result must not depend on where along the row the
maximum grows or by how much. §1 "Attention" formula: the softmax of a row is
unchanged when one constant is added to all of its scores.

  * key shift: K + 1 u^T leaves O (and the gradients) unchanged and moves lse
    by scale <q_i, u>;
  * equal V rows: O = v for every row, so dP = D and dS = 0: dQ = dK = 0 up to
    the fp32 rounding of two sums of the same products (a bound derived below);
  * rescale slack: the kernels move their reference maximum only when a tile's
    maximum exceeds it by more than 8 (log2 units). Keys are built so that the
    tile maxima of most rows rise by 7.9 (no move), 8.1 (move), 30 and 60, drop
    by 5 and 100, over 20 tiles of 64 keys and a ragged last one, at d = 64
    (the single-phase forward) and d = 128 with N >= 1024 (the ping-pong
    forward); forward and backward against the fp64 oracle, bf16 and fp16.

Inputs are built from exactly representable values so that the relations hold
exactly for the uploaded 16-bit data.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from attn_inputs import f32_to_bf16_bits, make_case
from gpu_helpers import TOL_BF16_O, TOL_GRAD_RELL2, check_lse, max_abs, rel_l2, term_rel_l2, to_f64
from oracle import (attention_bwd, attention_ds, attention_fwd, attention_probs, masked_attention_bwd,
                    masked_attention_ds, masked_attention_fwd)

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _round16(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values rounded to the 16-bit type (nearest even), as float64."""
    a32 = np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(a32).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).reshape(a32.shape).astype(np.float64)
    return a32.astype(np.float16).astype(np.float64)


def _upload(a: np.ndarray, dtype: str):
    """Exactly representable float64 values -> a device tensor of the 16-bit type (asserts exactness)."""
    import torch
    assert np.array_equal(_round16(a, dtype), a), "value not representable in the 16-bit type"
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


# ------------------------------------------------------------------ key shift


@pytest.mark.parametrize("dtype,N,d,umax", [("bf16", 333, 64, 50), ("f16", 333, 64, 50), ("bf16", 1100, 64, 50),
                                            ("bf16", 1100, 128, 50), ("f16", 1030, 128, 50),
                                            ("bf16", 333, 64, 8), ("bf16", 1100, 128, 8)])
def test_key_shift_invariance(gpu_lib, dtype, N, d, umax):
    """Forward and backward on (Q, K + 1 u^T, V) against the oracle on (Q, K, V): O and the gradients are those
    of the unshifted keys, lse is the unshifted one plus scale <q_i, u> (shifts of up to about 100 with
    |u_c| <= 50). K holds quarters in [-4, 4] and u quarters in [-umax, umax], so K + u (at most 8 significant
    bits) is exact.

    dQ = scale dS (K + 1 u^T) equals scale dS K only because every row of dS sums to 0; the kernels round dS to
    the 16-bit type (2^-9 relative) before that product, which leaves a row sum of order 2^-9 |dS_i| and adds it
    times u to dQ: the rounding error of dQ grows with |u| / |k|. So dQ is held to the workload tolerance by
    relative L2 for shifts up to 8 (about 5 times |k|), and for the large ones measured against the terms it
    sums, |scale| |dS| |K + 1 u^T| (term_rel_l2); dK = scale dS^T Q and dV = P^T dO do not involve the keys
    and are held to relative L2 at every shift."""
    import torch
    B, H = 1, 2
    x = make_case(B, H, N, d, dtype, seed=9100 + N + d)
    _say(f"key shift {dtype} B={B} H={H} N={N} d={d} |u| <= {umax}")
    rng = np.random.default_rng(N + d + umax)
    Q, V, DO = x.f64("q"), x.f64("v"), x.f64("do")
    K = np.clip(np.round(x.f64("k") * 4.0), -16, 16) / 4.0
    u = rng.integers(-4 * umax, 4 * umax + 1, size=(B, H, 1, d)) / 4.0
    Ks = K + u
    q, v, do = (_upload(a, dtype) for a in (Q, V, DO))
    ks = _upload(Ks, dtype)
    o, lse = gpu_lib.forward(q, ks, v, x.scale)
    dq, dk, dv = gpu_lib.backward(q, ks, v, o, lse, do, x.scale)
    torch.cuda.synchronize()
    ro, rl = attention_fwd(Q, K, V, x.scale)
    shift = x.scale * np.matmul(Q, np.swapaxes(u, -1, -2))[..., 0]
    _say(f"  lse shift range {shift.min():.1f} .. {shift.max():.1f}")
    assert max_abs(to_f64(o), ro) <= TOL_BF16_O
    e = check_lse(to_f64(lse), rl + shift, Q, Ks, x.scale, dtype)
    _say(f"  O max-abs {max_abs(to_f64(o), ro):.3e}, lse error / bound {e:.3f}")
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), attention_bwd(Q, K, V, DO, x.scale)):
        err = rel_l2(to_f64(got), ref)
        _say(f"  {name} rel-L2 {err:.3e}")
        if name != "dq" or umax <= 8:
            assert err <= TOL_GRAD_RELL2, name
        else:
            terms = abs(x.scale) * np.matmul(np.abs(attention_ds(Q, K, V, DO, x.scale)), np.abs(Ks))
            e_t = term_rel_l2(to_f64(got), ref, terms)
            _say(f"  dq error against its terms {e_t:.3e}")
            assert e_t <= TOL_GRAD_RELL2


# ------------------------------------------------------------------ equal V rows


@pytest.mark.parametrize("dtype,N,d,causal", [("bf16", 333, 64, False), ("bf16", 1100, 128, False),
                                              ("f16", 700, 64, False), ("bf16", 520, 64, True),
                                              ("bf16", 2048, 64, False)])
def test_equal_value_rows_give_zero_dq_dk(gpu_lib, dtype, N, d, causal):
    """All rows of V equal to one vector v: O_i = v, dP_ij = <dO_i, v> = D_i, so dS = 0 and dQ = dK = 0 exactly.
    The kernels form D_i from the stored O and dP_ij on the matrix cores, two fp32 sums of products; their
    difference is at most e_i = sum_c |dO_ic| |O_ic - v_c| + 3 gamma_(d+1) sum_c |dO_ic| (|v_c| + |O_ic|)
    (gamma_n = n u / (1 - n u), u = 2^-24). Hence |dQ_ic| <= |scale| e_i max_j |K_jc| and
    |dK_jc| <= |scale| sum_i P_ij e_i |Q_ic|, with 10 % slack for the 16-bit rounding of dS and of the
    recomputed weights. dV = P^T dO is checked against the oracle."""
    import torch
    B, H = 1, 2
    x = make_case(B, H, N, d, dtype, seed=9200 + N + d)
    _say(f"equal V rows {dtype} B={B} H={H} N={N} d={d} causal={causal}")
    Q, K, DO = x.f64("q"), x.f64("k"), x.f64("do")
    V = np.broadcast_to(x.f64("v")[:, :, :1, :], (B, H, N, d)).copy()
    q, k, v, do = (_upload(a, dtype) for a in (Q, K, V, DO))
    o, lse = gpu_lib.forward(q, k, v, x.scale, causal=causal)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, x.scale, causal=causal)
    torch.cuda.synchronize()
    O, gdq, gdk = to_f64(o), to_f64(dq), to_f64(dk)
    gamma = (d + 1) * U32 / (1 - (d + 1) * U32)
    e = (np.abs(DO) * np.abs(O - V)).sum(-1) + 3 * gamma * (np.abs(DO) * (np.abs(V) + np.abs(O))).sum(-1)
    if causal:
        P = np.stack([np.stack([masked_attention_probs(Q[b, h], K[b, h], x.scale) for h in range(H)])
                      for b in range(B)])
    else:
        P = attention_probs(Q, K, x.scale)
    bq = 1.1 * abs(x.scale) * e[..., None] * np.abs(K).max(axis=-2, keepdims=True)
    bk = 1.1 * abs(x.scale) * np.matmul(np.swapaxes(P, -1, -2), e[..., None] * np.abs(Q))
    _say(f"  O - v max {np.abs(O - V).max():.2e}; |dQ| max {np.abs(gdq).max():.2e} (bound max {bq.max():.2e}), "
         f"|dK| max {np.abs(gdk).max():.2e} (bound max {bk.max():.2e})")
    assert np.all(np.abs(gdq) <= bq) and np.all(np.abs(gdk) <= bk)
    if causal:
        rdv = masked_attention_bwd(Q, K, V, DO, x.scale, causal=True)[2]
    else:
        rdv = attention_bwd(Q, K, V, DO, x.scale)[2]
    assert rel_l2(to_f64(dv), rdv) <= TOL_GRAD_RELL2


def masked_attention_probs(q, k, scale):
    """Causal probabilities of one head from the masked oracle (V = I picks P out of O)."""
    n = k.shape[0]
    eye = np.eye(n)
    o, _ = masked_attention_fwd(q[None, None], k[None, None], eye[None, None], scale, causal=True)
    return o[0, 0]


# ------------------------------------------------------------------ rescale slack

TILE = 64  # keys per K/V tile of both 16-bit forward kernels
# Row maximum of each 64-key tile, in log2 units of the scaled score, for the designed rows: rises of 7.9 (below
# the slack: the reference stays), 8.1 (above: it moves), 30 and 60, drops of 5, 40 and 100, and a rise of 8.1
# in the ragged last tile (20 keys).
TILE_MAX = [0.0, 7.9, 7.9, 8.1, 38.1, 33.1, 46.0, 46.2, 6.2, 106.2, 114.3, 122.2, 22.2, 130.2, 130.3, 138.4,
            146.3, 154.4, 54.4, 162.5, 170.6]


def _slack_inputs(dtype: str, d: int, B: int = 1, H: int = 2, seed: int = 0, last: int = 20):
    """Q, K, V, dO (exact 16-bit values, float64) and the designed row mask.

    Designed rows (3 of every 4) carry q = (16, 1, noise); the others (0, 1, noise): their scores are small and
    they never rescale, so lanes of one wave disagree. Key j of tile t has k = (a_j, b_j, noise) with
    16 a_j + b_j the designed score: the tile's record key (at position 7 t mod the tile's length) scores
    TILE_MAX[t] / (scale log2 e), the others 1 to 12 log2 units less. Noise components ~ N(0, 1/1024) (about
    0.002 log2 units of score spread, so every tile maximum lands within 0.05 of its design)."""
    n_tiles = len(TILE_MAX)
    N = TILE * (n_tiles - 1) + last
    scale = float(np.float32(1.0 / math.sqrt(d)))
    c = scale * math.log2(math.e)
    rng = np.random.default_rng(seed + d)
    Q = _round16(rng.standard_normal((B, H, N, d)) / 32.0, dtype)
    K = _round16(rng.standard_normal((B, H, N, d)) / 32.0, dtype)
    designed = (np.arange(N) % 4) != 3
    Q[..., 0] = np.where(designed, 16.0, 0.0)
    Q[..., 1] = 1.0
    for t in range(n_tiles):
        lo, hi = t * TILE, min(N, (t + 1) * TILE)
        target = np.full((B, H, hi - lo), TILE_MAX[t]) - rng.uniform(1.0, 12.0, (B, H, hi - lo))
        target[..., (7 * t) % (hi - lo)] = TILE_MAX[t]
        score = target / c
        a = _round16(score / 16.0, dtype)
        K[..., lo:hi, 0] = a
        K[..., lo:hi, 1] = _round16(score - 16.0 * a, dtype)
    V = _round16(rng.standard_normal((B, H, N, d)), dtype)
    DO = _round16(rng.standard_normal((B, H, N, d)), dtype)
    return Q, K, V, DO, designed, scale


# The last tile holds 20 keys (ragged: the single-phase forward at d = 64) or 64 (whole tiles: the pipelined
# forward at d = 64, which takes the reference move only on its full path).
@pytest.mark.parametrize("dtype,d,causal,last", [("bf16", 64, False, 20), ("f16", 64, False, 20), ("bf16", 128, False, 20),
                                                 ("f16", 128, False, 20), ("bf16", 64, True, 20), ("bf16", 64, False, 64),
                                                 ("f16", 64, False, 64)])
def test_rescale_slack(gpu_lib, dtype, d, causal, last):
    import torch
    Q, K, V, DO, designed, scale = _slack_inputs(dtype, d, seed=9300, last=last)
    B, H, N, _ = Q.shape
    _say(f"rescale slack {dtype} B={B} H={H} N={N} d={d} causal={causal}")
    # The realised tile maxima of every designed row, from the oracle's exact probabilities, are the designed
    # ones: log2 P_ij = scale log2(e) s_ij - log2 l_i, so tile maxima of log2 P relative to tile 0 are those of
    # the scaled scores in log2 units.
    want = np.array(TILE_MAX) - TILE_MAX[0]
    for b in range(B):
        for h in range(H):
            lp = np.log2(attention_probs(Q[b, h][designed], K[b, h], scale))
            tmax = np.stack([lp[:, t * TILE:(t + 1) * TILE].max(axis=1) for t in range(len(TILE_MAX))], axis=1)
            dev = np.abs(tmax - tmax[:, :1] - want).max()
            assert dev <= 0.05, dev
    q, k, v, do = (_upload(a, dtype) for a in (Q, K, V, DO))
    o, lse = gpu_lib.forward(q, k, v, scale, causal=causal)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, scale, causal=causal)
    torch.cuda.synchronize()
    if causal:
        ro, rl = masked_attention_fwd(Q, K, V, scale, causal=True)
        rg = masked_attention_bwd(Q, K, V, DO, scale, causal=True)
    else:
        ro, rl = attention_fwd(Q, K, V, scale)
        rg = attention_bwd(Q, K, V, DO, scale)
    eo = max_abs(to_f64(o), ro)
    el = check_lse(to_f64(lse), rl, Q, K, scale, dtype)
    _say(f"  O max-abs {eo:.3e}, lse error / bound {el:.3f}")
    assert eo <= TOL_BF16_O
    # dQ = scale dS K and dK = scale dS^T Q sum terms with one large component (k_0 up to about 80, q_0 = 16)
    # beside components near 1/32, and the rows of dS sum to 0: those sums cancel, and their rounding error
    # (the 16-bit dS) is measured against the terms (term_rel_l2). dV = P^T dO is held to relative L2.
    ds = np.abs(masked_attention_ds(Q, K, V, DO, scale, causal=True) if causal else attention_ds(Q, K, V, DO, scale))
    terms = {"dq": abs(scale) * np.matmul(ds, np.abs(K)), "dk": abs(scale) * np.matmul(np.swapaxes(ds, -1, -2),
                                                                                       np.abs(Q))}
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
        err = rel_l2(to_f64(got), ref)
        if name == "dv":
            _say(f"  dv rel-L2 {err:.3e}")
            assert err <= TOL_GRAD_RELL2, name
        else:
            e_t = term_rel_l2(to_f64(got), ref, terms[name])
            _say(f"  {name} rel-L2 {err:.3e}, against its terms {e_t:.3e}")
            assert e_t <= TOL_GRAD_RELL2, name
