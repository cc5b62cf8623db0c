"""Host logic of bench.py that the recorded figures depend on: which kernel a shape runs (it names the roofline's
kernel and its traffic record), which instruction mix stands for it, and the FLOP counts (CPU only)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_forward_kernel_names():
    assert bench.fwd_kernel_name(4096, 64, False) == "fwd_sp_kernel"
    assert bench.fwd_kernel_name(196, 64, False) == "fwd_kernel"         # under 256 keys
    assert bench.fwd_kernel_name(4096, 64, True) == "fwd_sp_kernel"      # causal at d_k 64, 1024 keys or more
    assert bench.fwd_kernel_name(512, 64, True) == "fwd_kernel"          # causal at d_k 64, under 1024 keys
    assert bench.fwd_kernel_name(16384, 128, True) == "fwd_sp_kernel"    # causal at d_k 128: pipelined + diagonal
    assert bench.fwd_kernel_name(1100, 128, True) == "fwd_kernel"        # causal, not whole tiles
    assert bench.fwd_kernel_name(16384, 128, False) == "fwd_sp_kernel"   # whole tiles, 1024 keys or more
    assert bench.fwd_kernel_name(1100, 128, False) == "fwd_pp_kernel"    # not whole tiles
    assert bench.fwd_kernel_name(512, 128, False) == "fwd_kernel"
    assert bench.fwd_kernel_name(4096, 32, False) == "fwd_kernel"


def test_dkdv_kernel_names():
    assert bench.dkdv_kernel_name(4096, 64, False) == "bwd_dkdv_sp_kernel"
    assert bench.dkdv_kernel_name(196, 64, False) == "bwd_dkdv_sp_kernel"    # 4 steps, the last partial
    assert bench.dkdv_kernel_name(128, 64, False) == "bwd_dkdv_kernel"       # 2 steps: under the ring of 3
    assert bench.dkdv_kernel_name(129, 64, False) == "bwd_dkdv_sp_kernel"
    assert bench.dkdv_kernel_name(4096, 64, True) == "bwd_dkdv_sp_kernel"    # causal, whole 128-key blocks
    assert bench.dkdv_kernel_name(4032, 64, True) == "bwd_dkdv_kernel"       # causal, a partial key block
    assert bench.dkdv_kernel_name(4096, 128, False) == "bwd_dkdv_kernel"
    assert bench.fused_kernel_name(196, 64, False) == "bwd_dkdv_sp_dq_kernel"
    assert bench.fused_kernel_name(197, 64, True) == "bwd_dkdv_dq_kernel"
    assert bench.fused_kernel_name(256, 64, True) == "bwd_dkdv_dq_kernel"     # causal: single-phase bodies
    assert bench.fused_kernel_name(100, 64, False) == "bwd_dkdv_dq_kernel"
    assert bench.dq_kernel_name(8, 16, 4096, 64, False) == "bwd_dq_kernel"     # 2048 two-block workgroups
    assert bench.dq_kernel_name(4, 12, 2048, 64, False) == "bwd_dq_sp_kernel"  # 384
    assert bench.dq_kernel_name(4, 12, 2048, 64, True) == "bwd_dq_kernel"
    assert bench.dq_kernel_name(4, 12, 128, 64, False) == "bwd_dq_kernel"      # 2 tiles: under the ring of 3


def test_mix_of_kernel():
    from tiled_attention_08_amd.ceiling import MIXES
    for kernel, d, mix in (("bwd_dkdv_sp_kernel", 64, "dkdv"), ("bwd_dkdv_dq_kernel", 64, "dkdv"),
                           ("bwd_dkdv_sp_dq_kernel", 64, "dkdv"), ("bwd_dq_sp_kernel", 64, "dq"),
                           ("bwd_dq_kernel", 64, "dq"), ("fwd_sp_kernel", 64, "fwd64"), ("fwd_sp_kernel", 128, "fwd128"),
                           ("fwd_pp_kernel", 128, "fwd128")):
        assert bench.mix_of_kernel(kernel, d) == mix and mix in MIXES
    assert bench.mix_of_kernel("bwd_dkdv_kernel", 128) is None and bench.mix_of_kernel("fwd_kernel", 32) is None


def test_flop_counts():
    # 4 B H N^2 d forward, 10 B H N^2 d backward; causal counts the N (N + 1) / 2 visible pairs.
    assert bench.fwd_flops(8, 16, 4096, 64) == 4 * 8 * 16 * 4096 ** 2 * 64
    assert bench.bwd_flops(8, 16, 4096, 64) == 10 * 8 * 16 * 4096 ** 2 * 64
    assert bench.fwd_flops(1, 1, 4, 2, causal=True) == 4 * (4 * 5 // 2) * 2


def test_host_threads_reports_affinity():
    t = bench.host_threads()
    assert t["affinity_cores"] == len(os.sched_getaffinity(0)) and t["cores"] >= 1
