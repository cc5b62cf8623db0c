"""The seeded generator: determinism, bfloat16 rounding, workload shapes, planted keys."""
import math

import numpy as np
import pytest

from attn_inputs import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_case, make_inputs)


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even to bfloat16 agrees bit for bit with torch's CPU conversion."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40, 1e-38], dtype=np.float32),
        # exact ties: mantissa bit pattern ...1 1000... and ...0 1000...
        np.array([0x3F808000, 0x3F818000, 0x3F80C000], dtype=np.uint32).view(np.float32),
    ])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_determinism_and_seed_dependence():
    a = make_case(2, 3, 50, 64, "bf16", seed=5)
    b = make_case(2, 3, 50, 64, "bf16", seed=5)
    c = make_case(2, 3, 50, 64, "bf16", seed=6)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a.raw[n], b.raw[n])
        assert not np.array_equal(a.raw[n], c.raw[n])


def test_workload_table():
    """The five workloads: shapes, dtypes, passes and the fp32-rounded 1/sqrt(d_k) scale."""
    shapes = {w: (x.B, x.H, x.N, x.d, x.dtype) for w, x in WORKLOADS.items()}
    assert shapes == {1: (1, 1, 196, 64, "f32"), 2: (32, 12, 196, 64, "bf16"), 3: (8, 16, 4096, 64, "bf16"),
                      4: (2, 16, 16384, 128, "bf16"), 5: (4, 12, 2048, 64, "bf16")}
    assert WORKLOADS[4].passes == ("fwd",) and WORKLOADS[3].passes == ("fwd", "bwd")
    assert WORKLOADS[2].scale == 0.125
    assert WORKLOADS[4].scale == float(np.float32(1 / math.sqrt(128)))


def test_small_workload_inputs():
    x = make_inputs(1)
    assert x.dtype == "f32" and x.raw["q"].dtype == np.float32 and x.raw["q"].shape == (1, 1, 196, 64)
    assert "do" not in x.raw
    assert abs(x.raw["q"].std() - 1.0) < 0.05


def test_stress_distributions_and_planting():
    """Stress workload recipe on one reduced draw: Q,K ~ N(0, 64), V ~ U(-1,1), 1% planted copies."""
    x = make_case(1, 2, 2048, 64, "bf16", seed=0, wid=5, qk_sigma=8.0, v_dist="uniform", planted_frac=0.01)
    q, k, v = x.f64("q"), x.f64("k"), x.f64("v")
    assert abs(q.std() - 8.0) < 0.2 and abs(k.std() - 8.0) < 0.2
    assert v.min() >= -1.0 and v.max() <= 1.0 and abs(v.mean()) < 0.02
    assert x.planted.shape == (1, 2, 20, 2)
    for h in range(2):
        rows, keys = x.planted[0, h, :, 0], x.planted[0, h, :, 1]
        assert len(set(rows.tolist())) == 20 and len(set(keys.tolist())) == 20
        np.testing.assert_array_equal(x.raw["k"][0, h, keys], x.raw["q"][0, h, rows])


def test_f16_rounding_matches_torch():
    """fp16 cases round with numpy's float16 conversion (nearest even), the same as torch's CPU cast."""
    torch = pytest.importorskip("torch")
    x = make_case(1, 2, 50, 64, "f16", seed=9)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9, 0])))
    q32 = rng.standard_normal(size=(1, 2, 50, 64), dtype=np.float32)
    ref = torch.from_numpy(q32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(x.raw["q"], ref)
    np.testing.assert_array_equal(x.f64("q"), ref.view(np.float16).astype(np.float64))
