"""The instruction-mix probe (libattn_ceiling.so) runs on the GPU for every mix and reports a finite rate within
the chip's peak. It is measurement infrastructure beside the attention library, not part of its path."""
import math

import pytest

pytestmark = pytest.mark.gpu


def test_every_mix_runs():
    from tiled_attention_08_amd.ceiling import MIXES, mix_ceiling
    for mix in MIXES:
        print(f"mix {mix}", flush=True)
        r = mix_ceiling(mix, iters=200)
        assert math.isfinite(r["value"]) and 0 < r["value"] < 2516.6 * 1.05, r
