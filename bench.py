#!/usr/bin/env python3
"""Throughput of the fused attention path on one MI355X.

One step = the whole hot path over one batch of synthetic input: the fused
forward (attn_fwd) followed by the recompute-based backward (attn_bwd: delta, dK/dV
and dQ launches), on the long-sequence workload B=8, H=16, N=4096, d_k=64, bf16
(inputs seeded, already resident in device memory when timing starts).

    python bench.py [--steps K] [--warmup W] [--workload 1|2|3|4|5] [--causal] [--dtype bf16|f16]
                    [--cold] [--graph] [--no-cpu-baseline]
    python bench.py --workload 2 --proj      (the ViT block with its query/key/value projection)
    python bench.py --workload 2 --dtype f32 (fp32 storage and arithmetic, forward and backward)

Prints ONE JSON line on stdout; progress goes to stderr. FLOPs are
algorithmic: forward 4*B*H*N^2*d (Q K^T and P V), backward 10*B*H*N^2*d
(the Q K^T recompute, dP = dO V^T, dV = P^T dO, dK = dS^T Q, dQ = dS K); work
the implementation repeats (the dQ kernel's second Q K^T and dO V^T) is not
counted.

The "roofline" object describes the kernel that takes the most time per
step, timed on its own with HIP events over back-to-back launches on the
stream it runs on. "cpu_baseline" is the fp64 CPU oracle, timed on a bounded
sample of whole heads of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd+bwd (4·B·H·N²·d fwd) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def pairs(N, causal=False):
    """Query-key pairs of one head the method computes: N^2, or N(N+1)/2 under the causal mask."""
    return N * (N + 1) / 2.0 if causal else float(N) * N


def fwd_flops(B, H, N, d, causal=False):
    return 4.0 * B * H * pairs(N, causal) * d


def bwd_flops(B, H, N, d, causal=False):
    return 10.0 * B * H * pairs(N, causal) * d


def time_launches(fn, reps: int) -> float:
    """Average milliseconds per call of ``fn`` over ``reps`` back-to-back calls (HIP events on the current stream)."""
    import torch
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def sources_sha256() -> str:
    """sha256 over the attention library's kernel sources (csrc/attn_*.hip and *.h, sorted by path; the
    instruction-mix probe's source is not part of it)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "tiled_attention_08_amd", "csrc")
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(csrc, "attn_*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE / WRITE_SIZE record, or None
    if there is none for this workload or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["traffic_bytes"])


def fwd_kernel_name(N: int, d: int, causal: bool) -> str:
    """The forward kernel the library launches for a bf16/fp16 shape without key padding: the software-pipelined
    kernel for rows of whole 64-key tiles (at d_k 64 unmasked with 256 keys or more or causal with 1024 or more;
    unmasked or causal with 1024 or more at d_k 128), the ping-pong kernel for other unmasked rows of 1024 keys or
    more at d_k 128, the single-phase kernel otherwise."""
    if d == 64 and N % 64 == 0 and (N >= 1024 if causal else N >= 256):
        return "fwd_sp_kernel"
    if d == 128 and N % 64 == 0 and N >= 1024:
        return "fwd_sp_kernel"
    return "fwd_pp_kernel" if N >= 1024 and not causal and d == 128 else "fwd_kernel"


def dkdv_kernel_name(N: int, d: int, causal: bool) -> str:
    """The stand-alone dK/dV kernel for a shape without key padding: the software-pipelined kernel at d_k 64 for
    unmasked rows of at least three 64-query steps (the last may be partial) and for causal rows of whole 128-key
    blocks (N a multiple of 128, at least 256), the single-phase kernel otherwise."""
    if d == 64 and (N + 63) // 64 >= 3 and (not causal or N % 128 == 0):
        return "bwd_dkdv_sp_kernel"
    return "bwd_dkdv_kernel"


def dq_kernel_name(B: int, H: int, N: int, d: int, causal: bool) -> str:
    """The stand-alone dQ kernel for a shape without key padding: the software-pipelined kernel (one 32-query block
    per wave) for unmasked rows of at least three 64-key tiles at d_k 64 when the two-block kernel's grid would be
    under 4 workgroups per CU, the two-block single-phase kernel otherwise."""
    if d == 64 and not causal and (N + 63) // 64 >= 3 and B * H * ((N + 255) // 256) < 4 * 256:
        return "bwd_dq_sp_kernel"
    return "bwd_dq_kernel"


def fused_kernel_name(N: int, d: int, causal: bool) -> str:
    """The combined dK/dV + dQ launch for a shape without key padding: with the pipelined dK/dV body where the
    stand-alone pipelined kernel applies to unmasked rows, with the single-phase one otherwise (causal rows
    included)."""
    if not causal and dkdv_kernel_name(N, d, False) == "bwd_dkdv_sp_kernel":
        return "bwd_dkdv_sp_dq_kernel"
    return "bwd_dkdv_dq_kernel"


def mix_of_kernel(kernel: str, d: int):
    """The instruction mix (libattn_ceiling.so) a 16-bit kernel issues per product, where one was counted:
    d_k = 64 for the backward kernels and the d_k = 64 forward, d_k = 128 for the forward."""
    if d == 64:
        return {"bwd_dkdv_kernel": "dkdv", "bwd_dkdv_sp_kernel": "dkdv", "bwd_dkdv_dq_kernel": "dkdv",
                "bwd_dkdv_sp_dq_kernel": "dkdv", "bwd_dq_sp_kernel": "dq",
                "bwd_dq_kernel": "dq", "fwd_kernel": "fwd64", "fwd_sp_kernel": "fwd64"}.get(kernel)
    if d == 128:
        return {"fwd_kernel": "fwd128", "fwd_pp_kernel": "fwd128", "fwd_sp_kernel": "fwd128"}.get(kernel)
    return None


# Matrix-core work per unit of algorithmic work: the dQ kernel repeats the S and dP products (3 of its products
# per algorithmic one), the fused backward launch likewise (14 per 10).
MFMA_PER_ALGORITHMIC = {"bwd_dq_kernel": 3.0, "bwd_dq_sp_kernel": 3.0, "bwd_dkdv_dq_kernel": 1.4,
                        "bwd_dkdv_sp_dq_kernel": 1.4}


def attach_attainable(roofline: dict, d: int, causal: bool) -> None:
    """Adds the measured matrix-core ceiling of the kernel's instruction mix to an MFMA-bound roofline object:
    what that mix allows on this chip with random operands (see include/attn_ceiling.h), and the kernel's
    matrix-core rate as a fraction of it. "peak" and "frac" stay the published figure and the fraction of it.
    Not for causal launches, whose diagonal tiles do more products than the visible pairs count."""
    mix = mix_of_kernel(roofline["kernel"], d)
    if roofline.get("bound") != "mfma" or mix is None or causal:
        return
    from tiled_attention_08_amd.ceiling import mix_ceiling
    c = mix_ceiling(mix)
    rate = roofline["achieved"] * MFMA_PER_ALGORITHMIC.get(roofline["kernel"], 1.0)
    roofline["attainable"] = {**c, "kernel_mfma_rate": round(rate, 2), "frac": round(rate / c["value"], 4)}


def roofline_of(kernel: str, avg_ms: float, flops: float, nbytes: float, workload: str) -> dict:
    """The roofline object for one kernel: its bound follows from its algorithmic FLOP per algorithmic HBM byte
    (matrix cores at or above the machine balance 2516.6 TFLOP/s / 8 TB/s = 315, HBM below it)."""
    intensity = flops / nbytes
    t_s = avg_ms * 1e-3
    if intensity >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / t_s / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = nbytes / t_s / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBS, 4)}
    r.update({"traffic": measured_traffic(workload, kernel), "kernel": kernel, "avg_ms": round(avg_ms, 5),
              "algorithmic_bytes": nbytes, "flop_per_byte": round(intensity, 1)})
    return r


def host_threads() -> dict:
    """Threads the oracle runs on: "cores" = the BLAS pool's thread count (numpy's products are the only
    multi-threaded part), "affinity_cores" = len(os.sched_getaffinity(0)), the host cores this process may use."""
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [int(p.get("num_threads", 1)) for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:  # threadpoolctl missing: numpy's BLAS uses the affinity set
        blas = []
    threads = max(blas) if blas else affinity
    return {"cores": threads, "blas_threads": threads if blas else None, "affinity_cores": affinity}


def cpu_baseline(wid: int, seed: int, budget_s: float, causal: bool = False) -> dict:
    """The fp64 oracle (forward + backward) on whole heads of the workload, for about ``budget_s`` seconds."""
    import numpy as np
    from attn_inputs import WORKLOADS, make_inputs
    from oracle import attention_bwd, attention_fwd, masked_attention_bwd, masked_attention_fwd
    w = WORKLOADS[wid]
    x = make_inputs(wid, seed=seed)
    heads, elapsed = 0, 0.0
    order = [(b, h) for b in range(w.B) for h in range(w.H)]
    while heads < len(order) and (heads == 0 or elapsed * (heads + 1) / heads <= budget_s):
        b, h = order[heads]
        Q, K, V = (x.f64(n, (b, h)) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        if causal:
            Q, K, V = Q[None, None], K[None, None], V[None, None]
            masked_attention_fwd(Q, K, V, x.scale, causal=True)
            if "bwd" in w.passes:
                masked_attention_bwd(Q, K, V, x.f64("do", (b, h))[None, None], x.scale, causal=True)
        else:
            attention_fwd(Q, K, V, x.scale)
            if "bwd" in w.passes:
                attention_bwd(Q, K, V, x.f64("do", (b, h)), x.scale)
        elapsed += time.perf_counter() - t0
        heads += 1
    flops = (fwd_flops(1, heads, w.N, w.d, causal) + (bwd_flops(1, heads, w.N, w.d, causal) if "bwd" in w.passes else 0.0))
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", **host_threads(), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of the same workload ({'+'.join(w.passes)}{', causal' if causal else ''}, fp64, full N x N per head), "
                      f"{elapsed:.1f} s", "seconds": round(elapsed, 3)}


PEAK_F32_TFLOPS = 157.3  # MI355X fp32 vector ALU


def bench_f32(args, w) -> int:
    """fp32 forward (attn_fwd_f32) of a forward-only fp32 workload: latency per launch and fp32 vector-ALU roofline."""
    import numpy as np
    import torch
    from attn_inputs import make_inputs
    from tiled_attention_08_amd import _lib as attn
    B, H, N, d = w.B, w.H, w.N, w.d
    x = make_inputs(w.wid, seed=args.seed)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x.raw[n])).cuda() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    def step():  # on the current stream: the capture stream while the graph below is recorded
        attn.attn_fwd_f32(q, k, v, o, lse, x.scale, torch.cuda.current_stream())

    step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # Back-to-back calls through the binding: for a kernel this small the host's per-call work (argument checks)
    # sets the pace, so this figure depends on the host CPU; reported beside the value.
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    host_ms = t0.elapsed_time(t1) / args.steps
    # The value: one HIP graph holding the K launches, replayed once (the launches run back to back on the GPU
    # with no host work between them).
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(args.steps):
            step()
    g.replay()
    torch.cuda.synchronize()
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    flops = fwd_flops(B, H, N, d)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] fp32 forward {ms * 1e3:.2f} us per launch in a graph ({host_ms * 1e3:.2f} us per call from the "
        f"host), {value:.3f} TFLOP/s")
    record = {
        "metric": "attention forward latency, fp32 (us per launch)", "value": round(ms * 1e3, 3), "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d_k": d, "passes": "fwd"},
        "tflops": round(value, 4), "timing": f"{args.steps} launches captured in one HIP graph, replayed once",
        "host_call_us": round(host_ms * 1e3, 3),
        "roofline": {"bound": "alu", "achieved": round(value, 4), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_F32_TFLOPS, 5), "traffic": None, "kernel": "fwd_f32_kernel",
                     "avg_ms": round(ms, 5),
                     "note": "one head of 196 rows: 25 workgroups of 8 rows on 256 CUs, so latency dominates"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(w.wid, args.seed, min(args.cpu_seconds, 2.0))
    print(json.dumps(record), flush=True)
    return 0


def bench_f32_train(args, w) -> int:
    """fp32 storage and arithmetic (attn_fwd_f32 + attn_bwd_f32) on a workload with a backward: TFLOP/s of the
    step against the fp32 vector-ALU peak (the fp32 kernels run on the vector ALU, not the matrix cores)."""
    import numpy as np
    import torch
    from attn_inputs import make_case
    from tiled_attention_08_amd import _lib as attn
    B, H, N, d = w.B, w.H, w.N, w.d
    log(f"[bench] workload {w.wid} {w.name} in fp32: B={B} H={H} N={N} d={d}, seed {args.seed}")
    x = make_case(B, H, N, d, "f32", seed=args.seed, wid=w.wid, qk_sigma=w.qk_sigma, v_dist=w.v_dist,
                  planted_frac=w.planted_frac)
    q, k, v, do = (torch.from_numpy(np.ascontiguousarray(x.raw[n])).cuda() for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = attn.workspace_for(q)
    stream = torch.cuda.current_stream()

    def fwd():
        attn.attn_fwd_f32(q, k, v, o, lse, x.scale, stream)

    def bwd():
        attn.attn_bwd_f32(q, k, v, o, lse, do, dq, dk, dv, x.scale, ws, stream)

    def step():
        fwd()
        bwd()

    step()
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        if not torch.isfinite(t).all():
            log("[bench] non-finite output")
            return 1
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    flops = fwd_flops(B, H, N, d) + bwd_flops(B, H, N, d)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] fp32 {ms:.4f} ms/step, {value:.2f} TFLOP/s")
    reps = args.kernel_reps
    # The forward is one kernel; the fp32 backward (delta, dK/dV, dQ) is timed as its three launches together.
    kernels = {"fwd_f32": time_launches(fwd, reps), "bwd_f32": time_launches(bwd, reps)}
    log("[bench] kernel ms: " + ", ".join(f"{kn} {t:.4f}" for kn, t in kernels.items()))
    kflops = {"fwd_f32": fwd_flops(B, H, N, d), "bwd_f32": bwd_flops(B, H, N, d)}
    names = {"fwd_f32": "fwd_f32_kernel",
             "bwd_f32": "attn_bwd_f32 (bwd_prep_f32_kernel, bwd_dkdv_f32_kernel, bwd_dq_f32_kernel)"}
    dominant = max(kernels, key=kernels.get)
    achieved = kflops[dominant] / (kernels[dominant] * 1e-3) / 1e12
    record = {
        "metric": "attention TFLOP/s fwd+bwd in fp32 (vector ALU) and % of MI355X fp32 vector peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + "_f32", "B": B, "H": H, "N": N, "d_k": d, "passes": "fwd+bwd",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "frac_of_f32_vector_peak": round(value / PEAK_F32_TFLOPS, 4),
        "kernel_ms": {kn: round(t, 5) for kn, t in kernels.items()},
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F32_TFLOPS, 4), "traffic": None, "kernel": names[dominant],
                     "avg_ms": round(kernels[dominant], 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(w.wid, args.seed, args.cpu_seconds)
    print(json.dumps(record), flush=True)
    return 0


def proj_flops(B, N, D, H, d):
    """One product of the query/key/value projection: 2 * tokens * D * 3 H d (the forward has one, the backward two)."""
    return 2.0 * B * N * D * 3 * H * d


def cpu_baseline_block(B, N, D, H, d, seed: int, budget_s: float) -> dict:
    """The fp64 oracle on whole images of the ViT block (projection, attention, their backward), ~budget_s seconds."""
    from attn_inputs import make_case, make_proj_case
    from oracle import attention_bwd, attention_fwd, qkv_projection, qkv_projection_bwd, split_qkv
    import numpy as np
    c = make_proj_case(B, N, D, H, d, "bf16", seed=seed, wid=2)
    g = make_case(B, H, N, d, "bf16", seed=seed, wid=2)
    X, W, DO = c.f64("x"), c.f64("w"), g.f64("do")
    scale = g.scale
    imgs, elapsed = 0, 0.0
    while imgs < B and (imgs == 0 or elapsed * (imgs + 1) / imgs <= budget_s):
        t0 = time.perf_counter()
        x1 = X[imgs:imgs + 1]
        q, k, v = split_qkv(qkv_projection(x1, W))
        dqkv = np.empty((1, N, 3, H, d))
        for h in range(H):
            attention_fwd(q[0, h], k[0, h], v[0, h], scale)
            gq, gk, gv = attention_bwd(q[0, h], k[0, h], v[0, h], DO[imgs, h], scale)
            dqkv[0, :, 0, h], dqkv[0, :, 1, h], dqkv[0, :, 2, h] = gq, gk, gv
        qkv_projection_bwd(x1, W, dqkv)
        elapsed += time.perf_counter() - t0
        imgs += 1
    flops = imgs * (3 * proj_flops(1, N, D, H, d) + fwd_flops(1, H, N, d) + bwd_flops(1, H, N, d))
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", **host_threads(), "kind": "oracle",
            "sample": f"{imgs} of {B} images of the same block (projection, attention and their backward, fp64), "
                      f"{elapsed:.1f} s", "seconds": round(elapsed, 3)}


def bench_proj(args, w) -> int:
    """ViT attention block: query/key/value projection, attention in the packed layout, and both backward passes."""
    import numpy as np
    import torch
    from attn_inputs import make_case, make_proj_case
    from tiled_attention_08_amd import _lib as attn
    B, H, N, d = w.B, w.H, w.N, w.d
    D = H * d
    log(f"[bench] ViT block with projection: B={B} N={N} D={D} H={H} d={d} bf16, seed {args.seed}")
    c = make_proj_case(B, N, D, H, d, "bf16", seed=args.seed, wid=w.wid)
    g = make_case(B, H, N, d, "bf16", seed=args.seed, wid=w.wid)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    x, wt = up(c.raw["x"]), up(c.raw["w"])
    do = up(g.raw["do"]).transpose(1, 2).contiguous()                       # [B, N, H, d]
    qkv = torch.empty((B, N, 3, H, d), dtype=torch.bfloat16, device="cuda")
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dqkv = torch.empty_like(qkv)
    dq, dk, dv = dqkv[:, :, 0], dqkv[:, :, 1], dqkv[:, :, 2]
    dx, dw = torch.empty_like(x), torch.empty_like(wt)
    ws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    pws = attn.proj_workspace_for(x, wt)
    scale = g.scale
    stream = torch.cuda.current_stream()

    def proj_fwd():
        attn.attn_qkv_proj(x, wt, qkv, stream)

    def att_fwd():
        attn.attn_fwd_ex(q, k, v, o, lse, scale, stream=stream, layout="qkv_packed")

    def att_bwd_stage(i):
        return lambda: attn.attn_bwd_stage(i, q, k, v, o, lse, do, dq, dk, dv, scale, ws, stream=stream,
                                           layout="qkv_packed")

    def att_bwd():
        attn.attn_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, scale, ws, stream=stream, layout="qkv_packed")

    def proj_bwd():
        attn.attn_qkv_proj_bwd(x, wt, dqkv, dx, dw, pws, stream)

    def step():
        proj_fwd()
        att_fwd()
        att_bwd()
        proj_bwd()

    step()
    torch.cuda.synchronize()
    for t in (qkv, o, lse, dqkv, dx, dw):
        if not torch.isfinite(t.float()).all():
            log("[bench] non-finite output")
            return 1
    for _ in range(args.warmup):
        step()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    pf = proj_flops(B, N, D, H, d)
    flops = 3 * pf + fwd_flops(B, H, N, d) + bwd_flops(B, H, N, d)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.4f} ms/step, {value:.1f} TFLOP/s")

    reps = args.kernel_reps
    fused = attn.attn_bwd_fused(B, H, N, d)
    kernels = {"proj_fwd": time_launches(proj_fwd, reps), "fwd": time_launches(att_fwd, reps),
               "bwd_prep": time_launches(att_bwd_stage(0), reps)}
    if fused:
        kernels["bwd_dkdv_dq"] = time_launches(att_bwd_stage(3), reps)
    else:
        kernels["bwd_dkdv"] = time_launches(att_bwd_stage(1), reps)
        kernels["bwd_dq"] = time_launches(att_bwd_stage(2), reps)
    kernels["proj_bwd"] = time_launches(proj_bwd, reps)
    log("[bench] kernel ms: " + ", ".join(f"{kname} {t:.4f}" for kname, t in kernels.items()))
    T, E, R, sz = B * N, B * H * N * d, B * H * N, 2
    kflops = {"proj_fwd": pf, "proj_bwd": 2 * pf, "fwd": fwd_flops(B, H, N, d), "bwd_prep": 0.0,
              "bwd_dkdv": 0.8 * bwd_flops(B, H, N, d), "bwd_dq": 0.2 * bwd_flops(B, H, N, d),
              "bwd_dkdv_dq": bwd_flops(B, H, N, d)}
    kbytes = {"proj_fwd": (T * D + D * 3 * H * d + T * 3 * H * d) * sz,
              "proj_bwd": (2 * T * D + 2 * D * 3 * H * d + T * 3 * H * d) * sz,
              "fwd": 4 * E * sz + 4 * R, "bwd_prep": 2 * E * sz + 12 * R, "bwd_dkdv": 6 * E * sz + 8 * R,
              "bwd_dq": 5 * E * sz + 8 * R, "bwd_dkdv_dq": 7 * E * sz + 8 * R}
    kname_full = {"proj_fwd": "gemm256_kernel", "proj_bwd": "attn_qkv_proj_bwd (dx and dw products, split sums)",
                  "fwd": fwd_kernel_name(N, d, False), "bwd_prep": "bwd_prep_kernel", "bwd_dkdv": dkdv_kernel_name(N, d, False),
                  "bwd_dq": dq_kernel_name(B, H, N, d, False), "bwd_dkdv_dq": fused_kernel_name(N, d, False)}
    # The roofline describes the longest single kernel (the projection backward is a group of launches).
    single = {kn: t for kn, t in kernels.items() if kn != "proj_bwd"}
    dominant = max(single, key=single.get)
    wkey = "vit_b16_block_with_qkv_projection"
    roofline = roofline_of(kname_full[dominant], kernels[dominant], kflops[dominant], kbytes[dominant], wkey)
    record = {
        "metric": "ViT attention block TFLOP/s fwd+bwd: query/key/value projection (3 products of 2*B*N*D*3*H*d) "
                  "plus attention (14*B*H*N^2*d), and % of MI355X bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wkey, "B": B, "N": N, "D": D, "H": H, "d_k": d, "passes": "fwd+bwd",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "frac_of_bf16_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {kn: round(t, 5) for kn, t in kernels.items()},
        "proj_tflops": {"fwd": round(pf / (kernels["proj_fwd"] * 1e-3) / 1e12, 2),
                        "bwd": round(2 * pf / (kernels["proj_bwd"] * 1e-3) / 1e12, 2)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        record["cpu_baseline"] = cpu_baseline_block(B, N, D, H, d, args.seed, args.cpu_seconds)
    print(json.dumps(record), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3, choices=(1, 2, 3, 4, 5),
                    help="3 = long sequence, the headline; 1 (fp32) and 4 run the forward only (their workloads have "
                         "no backward)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel-reps", type=int, default=20, help="launches per kernel for the roofline timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", default="bf16", choices=("bf16", "f16", "f32"),
                    help="storage type of Q, K, V, O and the gradients (f16 runs attn_fwd_ex / attn_bwd_ex; f32 runs "
                         "the fp32 forward and backward, vector ALU)")
    ap.add_argument("--cold", action="store_true",
                    help="rotate through copies of the inputs (about 1 GiB in all) so that every launch reads its "
                         "inputs from HBM, not from L2 or the MALL")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (forward + backward launches) in a HIP graph and time graph replays")
    ap.add_argument("--causal", action="store_true",
                    help="time the causal-mask path (attn_fwd_ex / attn_bwd_ex); FLOPs count the N(N+1)/2 visible "
                         "query-key pairs of each head")
    ap.add_argument("--proj", action="store_true",
                    help="with --workload 2: time the ViT attention block including the query/key/value projection "
                         "(D = H d_k) and its backward, attention in the packed layout")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the instruction-mix probe that adds the roofline's 'attainable' object")
    ap.add_argument("--mix-ceiling", action="store_true",
                    help="only run the instruction-mix probe (libattn_ceiling.so) for every mix and print one JSON "
                         "line: the sustained matrix-core rate each kernel's mix allows")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (three times) and exit: the "
                         "known-size reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args(argv)
    if args.mix_ceiling:
        from tiled_attention_08_amd.ceiling import MIXES, mix_ceiling
        res = {m: mix_ceiling(m) for m in MIXES}
        print(json.dumps({"metric": "sustained bf16 matrix-core rate per instruction mix", "unit": "TFLOP/s",
                          "peak": PEAK_BF16_TFLOPS,
                          "mixes": {m: {**r, "frac_of_peak": round(r["value"] / PEAK_BF16_TFLOPS, 4)}
                                    for m, r in res.items()}}), flush=True)
        return 0
    if args.copy_calibration_mib:
        import torch
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration_mib} MiB x 3")
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this attention library has no multi-GPU path "
              "(heads shard across GPUs with no communication; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from attn_inputs import WORKLOADS, make_case, make_inputs
    from tiled_attention_08_amd import _lib as attn

    w = WORKLOADS[args.workload]
    B, H, N, d = w.B, w.H, w.N, w.d
    cz = args.causal
    if w.dtype == "f32":
        return bench_f32(args, w)
    if args.dtype == "f32":
        if "bwd" not in w.passes or args.causal or args.cold or args.graph or args.proj:
            log("[bench] --dtype f32 times the fp32 forward and backward of a workload with a backward, no other mode")
            return 2
        return bench_f32_train(args, w)
    if args.proj:
        if args.workload != 2 or args.causal or args.dtype != "bf16" or args.cold or args.graph:
            log("[bench] --proj times the ViT-B/16 block: use it with --workload 2 only (bf16, no other mode)")
            return 2
        return bench_proj(args, w)
    log(f"[bench] workload {w.wid} {w.name}: B={B} H={H} N={N} d={d} {args.dtype}{' causal' if cz else ''}, seed {args.seed}")
    if args.dtype == "bf16":
        x = make_inputs(args.workload, seed=args.seed)
    else:
        x = make_case(B, H, N, d, args.dtype, seed=args.seed, wid=w.wid, qk_sigma=w.qk_sigma, v_dist=w.v_dist,
                      planted_frac=w.planted_frac, with_grad="bwd" in w.passes)

    def up(name):
        a = np.ascontiguousarray(x.raw[name])
        if args.dtype == "f16":
            return torch.from_numpy(a.view(np.float16)).cuda()
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    with_bwd = "bwd" in w.passes

    def new_set(src=None):
        t = {n: (up(n) if src is None else src[n].clone()) for n in ("q", "k", "v") + (("do",) if with_bwd else ())}
        t["o"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        if with_bwd:
            t.update(dq=torch.empty_like(t["q"]), dk=torch.empty_like(t["q"]), dv=torch.empty_like(t["q"]),
                     ws=attn.workspace_for(t["q"]))
        return t

    sets = [new_set()]
    set_bytes = sum(t.numel() * t.element_size() for t in sets[0].values())
    if args.cold:
        # Copies of the same inputs at other addresses, about 1 GiB in all (L2 4 MB per XCD, MALL 256 MB), used
        # in turn so that no launch finds its inputs in a cache.
        while len(sets) * set_bytes < (1 << 30) or len(sets) < 2:
            sets.append(new_set(sets[0]))
        log(f"[bench] cold: {len(sets)} input sets of {set_bytes / 2**20:.1f} MiB")
    scale = x.scale
    stream = torch.cuda.current_stream()
    turn = [0]

    def next_set():
        t = sets[turn[0] % len(sets)]
        turn[0] += 1
        return t

    def step():
        t = next_set()
        cs = torch.cuda.current_stream()  # the capture stream while a graph is recorded
        if args.causal or args.dtype != "bf16":
            attn.attn_fwd_ex(t["q"], t["k"], t["v"], t["o"], t["lse"], scale, causal=cz, stream=cs)
            if with_bwd:
                attn.attn_bwd_ex(t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"], t["dk"], t["dv"], scale,
                                 t["ws"], causal=cz, stream=cs)
            return
        attn.attn_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], scale, cs)
        if with_bwd:
            attn.attn_bwd(t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"], t["dk"], t["dv"], scale,
                          t["ws"], cs)

    # One checked step first, so that the host-side check does not leave the
    # GPU idle (and its clock low) between the warm-up and the timed steps.
    for _ in range(len(sets)):
        step()
    torch.cuda.synchronize()
    for st in sets:
        for n in ("o", "lse") + (("dq", "dk", "dv") if with_bwd else ()):
            if not torch.isfinite(st[n].float()).all():
                log("[bench] non-finite output")
                return 1
    for _ in range(args.warmup):
        step()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    if args.graph:
        # One graph per input set (each holds its own tensors); a step replays the next one.
        torch.cuda.synchronize()
        graphs = []
        for _ in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            graphs.append(g)
        gturn = [0]

        def step():  # noqa: F811  (the timed step becomes a graph replay)
            graphs[gturn[0] % len(graphs)].replay()
            gturn[0] += 1

        for _ in range(args.warmup):
            step()

    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    flops = fwd_flops(B, H, N, d, cz) + (bwd_flops(B, H, N, d, cz) if with_bwd else 0.0)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/step, {value:.1f} TFLOP/s")

    # Per-kernel timing (each kernel alone, back-to-back launches on the same stream).
    reps = args.kernel_reps
    def stage(i):
        def run():
            t = next_set()
            attn.attn_bwd_stage(i, t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"], t["dk"], t["dv"], scale,
                                t["ws"], causal=cz, stream=stream)
        return run

    def fwd_only():
        t = next_set()
        attn.attn_fwd_ex(t["q"], t["k"], t["v"], t["o"], t["lse"], scale, causal=cz, stream=stream)

    # The kernels the step launches: forward, delta, and either one combined dK/dV + dQ launch (stage 3, where
    # attn_bwd_fused says so) or the dK/dV and dQ kernels; the separate two are timed in both cases.
    fused = with_bwd and attn.attn_bwd_fused(B, H, N, d)
    kernels = {"fwd": time_launches(fwd_only, reps)}
    separate = {}
    if with_bwd:
        kernels["bwd_prep"] = time_launches(stage(0), reps)
        separate = {"bwd_dkdv": time_launches(stage(1), reps), "bwd_dq": time_launches(stage(2), reps)}
        if fused:
            kernels["bwd_dkdv_dq"] = time_launches(stage(3), reps)
        else:
            kernels.update(separate)
    log("[bench] kernel ms: " + ", ".join(f"{kname} {t:.4f}" for kname, t in {**kernels, **separate}.items()))
    # Algorithmic FLOPs per launch. The dK/dV kernel performs the S recompute,
    # dP, dV and dK products (8 B H N^2 d). The dQ kernel repeats S and dP to
    # avoid a cross-workgroup reduction; only its dQ product (2 B H N^2 d) is
    # algorithmic work, so its roofline fraction counts that alone. The combined
    # launch counts the whole backward (10 B H N^2 d).
    kflops = {"fwd": fwd_flops(B, H, N, d, cz), "bwd_dkdv": 0.8 * bwd_flops(B, H, N, d, cz),
              "bwd_dq": 0.2 * bwd_flops(B, H, N, d, cz), "bwd_prep": 0.0, "bwd_dkdv_dq": bwd_flops(B, H, N, d, cz)}
    # Algorithmic HBM bytes per launch: every tensor read or written once (E elements of s bytes per [B,H,N,d]
    # tensor, R fp32 rows per statistic).
    E, R, sz = B * H * N * d, B * H * N, 2
    kbytes = {"fwd": 4 * E * sz + 4 * R, "bwd_prep": 2 * E * sz + 12 * R, "bwd_dkdv": 6 * E * sz + 8 * R,
              "bwd_dq": 5 * E * sz + 8 * R, "bwd_dkdv_dq": 7 * E * sz + 8 * R}
    kname_full = {"fwd": fwd_kernel_name(N, d, cz), "bwd_dkdv": dkdv_kernel_name(N, d, cz),
                  "bwd_dq": dq_kernel_name(B, H, N, d, cz),
                  "bwd_prep": "bwd_prep_kernel", "bwd_dkdv_dq": fused_kernel_name(N, d, cz)}
    dominant = max(kernels, key=kernels.get)
    wkey = w.name + ("_causal" if cz else "") + ("_f16" if args.dtype == "f16" else "")
    roofline = roofline_of(kname_full[dominant], kernels[dominant], kflops[dominant], kbytes[dominant], wkey)
    if not args.no_ceiling:
        attach_attainable(roofline, d, cz)
    if args.cold:
        roofline["inputs"] = f"rotating {len(sets)} input sets ({set_bytes * len(sets) / 2**30:.2f} GiB, beyond L2 and MALL)"

    record = {
        "metric": METRIC if not cz else METRIC + ", causal mask (N(N+1)/2 pairs per head)", "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": wkey + ("_cold" if args.cold else "") + ("_graph" if args.graph else ""), "B": B, "H": H, "N": N, "d_k": d, "passes": "+".join(w.passes),
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "frac_of_bf16_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {kname: round(t, 5) for kname, t in kernels.items()},
        "bwd_fused": bool(fused),
        "kernel_ms_separate": {kname: round(t, 5) for kname, t in separate.items()} if fused else None,
        "fwd_tflops": round(fwd_flops(B, H, N, d, cz) / (kernels["fwd"] * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        record["cpu_baseline"] = cpu_baseline(args.workload, args.seed, args.cpu_seconds, cz)
    print(json.dumps(record), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
