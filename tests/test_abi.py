"""The C ABI on the host: the library loads, exports what include/attn.h declares, and
rejects bad arguments before launching anything.

No call here reaches a kernel launch: every call below fails exactly one
validation check, and the checks run on the host before any HIP call, so these
tests need no GPU. The fake device addresses are never dereferenced.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def L():
    from tiled_attention_08_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["attn_fwd", "attn_fwd_f32", "attn_fwd_ex", "attn_bwd", "attn_bwd_f32",
                                           "attn_bwd_ex", "attn_bwd_stage", "attn_bwd_ex_noalloc", "attn_bwd_fused",
                                           "attn_bwd_workspace_bytes", "attn_qkv_proj", "attn_qkv_proj_bwd",
                                           "attn_qkv_proj_bwd_workspace_bytes", "attn_status_string"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L.lib, name), name
        assert callable(getattr(L, name, None)), f"no Python wrapper for {name}"
    assert sorted(L.EXPORTS) == declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4):
        assert L.attn_status_string(code) and L.attn_status_string(code) != "unknown status"
    assert L.attn_status_string(7) == "unknown status"


# Distinct, 16-byte aligned fake device addresses, far apart (no overlaps).
A = [0x10_0000_0000 * (i + 1) for i in range(12)]


def fwd(L, *, q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=1, H=1, N=8, d=64, scale=0.125):
    return L.lib.attn_fwd(q, k, v, o, lse, B, H, N, d, scale, None)


def fwd_ex(L, *, dtype=0, layout=0, causal=0, kv_len=None, **kw):
    a = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=1, H=1, N=8, d=64, scale=0.125)
    a.update(kw)
    return L.lib.attn_fwd_ex(dtype, layout, a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                             a["scale"], causal, kv_len, None)


def fwd32(L, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=1, H=1, N=8, d=64, scale=0.125)
    args.update(kw)
    return L.lib.attn_fwd_f32(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"],
                              args["N"], args["d"], args["scale"], None)


def bwd(L, stage=None, ex=False, dtype=0, layout=0, causal=0, kv_len=None, **kw):
    a = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], do=A[5], dq=A[6], dk=A[7], dv=A[8], B=1, H=1, N=8, d=64,
             scale=0.125, ws=A[9], ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = L.attn_bwd_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
    head = (a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["N"],
            a["d"], a["scale"])
    tail = (a["ws"], a["ws_bytes"], None)
    if stage is None and not ex:
        return L.lib.attn_bwd(*head, *tail)
    if stage is None:
        return L.lib.attn_bwd_ex(dtype, layout, *head, causal, kv_len, *tail)
    return L.lib.attn_bwd_stage(stage, dtype, layout, *head, causal, kv_len, *tail)


def test_forward_rejections(L):
    INV, UNS = L.ATTN_ERR_INVALID_ARG, L.ATTN_ERR_UNSUPPORTED
    for f in (fwd, fwd32):
        assert f(L, q=None) == INV
        assert f(L, lse=None) == INV
        assert f(L, v=A[2] + 8) == INV                    # misaligned
        assert f(L, B=0) == INV and f(L, H=-1) == INV and f(L, N=0) == INV
        assert f(L, scale=float("nan")) == INV and f(L, scale=float("inf")) == INV
        assert f(L, d=80) == UNS and f(L, d=16) == UNS and f(L, d=256) == UNS and f(L, d=48) == UNS
        assert f(L, o=A[0]) == INV                        # output aliases an input
        assert f(L, o=A[0] + 16) == INV                   # partial overlap
        assert f(L, lse=A[3] + 64) == INV                 # lse inside o
        assert f(L, N=1 << 30) == UNS                     # beyond 32-bit per-head indexing


def test_extended_forward_rejections(L):
    INV, UNS = L.ATTN_ERR_INVALID_ARG, L.ATTN_ERR_UNSUPPORTED
    assert fwd_ex(L, dtype=2) == UNS and fwd_ex(L, dtype=-1) == UNS
    assert fwd_ex(L, causal=2) == INV and fwd_ex(L, causal=-1) == INV
    assert fwd_ex(L, kv_len=A[10] + 2) == INV               # kv_len not 4-byte aligned
    assert fwd_ex(L, kv_len=A[3] + 4) == INV                # kv_len inside o
    assert fwd_ex(L, kv_len=A[4]) == INV                    # kv_len on lse
    assert fwd_ex(L, q=None, causal=1) == INV
    assert fwd_ex(L, d=72, causal=1) == UNS
    assert fwd_ex(L, layout=3) == UNS and fwd_ex(L, layout=-1) == UNS


def test_layout_rejections(L):
    """Packed Q/K/V: k and v must sit H*d and 2*H*d elements after q; outputs may not touch the packed buffer."""
    INV = L.ATTN_ERR_INVALID_ARG
    B, H, N, d = 1, 2, 8, 64
    hd = H * d * 2                         # bytes between q, k and v inside one packed row
    qkv_bytes = 3 * B * N * H * d * 2
    good = dict(q=A[0], k=A[0] + hd, v=A[0] + 2 * hd, B=B, H=H, N=N, d=d)
    assert fwd_ex(L, layout=2, **dict(good, k=A[1])) == INV                    # k not inside q's packed row
    assert fwd_ex(L, layout=2, **dict(good, v=A[0] + hd)) == INV               # v == k
    assert fwd_ex(L, layout=2, **dict(good, o=A[0] + qkv_bytes - 256)) == INV  # o inside the packed buffer
    assert fwd_ex(L, layout=2, **dict(good, lse=A[0] + 2 * hd + 64)) == INV    # lse inside the packed buffer
    for stage in (None, 1):
        gq = dict(dq=A[6], dk=A[6] + hd, dv=A[6] + 2 * hd)
        assert bwd(L, stage, ex=True, layout=2, **dict(good, **dict(gq, dk=A[7]))) == INV    # dk not packed
        assert bwd(L, stage, ex=True, layout=2, **dict(good, **dict(gq, dq=A[0] + 16 * hd, dk=A[0] + 17 * hd,
                                                                       dv=A[0] + 18 * hd))) == INV  # grads on inputs


def test_backward_rejections(L):
    INV, UNS, WS = L.ATTN_ERR_INVALID_ARG, L.ATTN_ERR_UNSUPPORTED, L.ATTN_ERR_WORKSPACE
    for stage in (None, 0, 1, 2, 3):
        assert bwd(L, stage, dq=None) == INV
        assert bwd(L, stage, do=A[5] + 4) == INV
        assert bwd(L, stage, d=80) == UNS and bwd(L, stage, d=160) == UNS
        assert bwd(L, stage, ws=None) == WS
        assert bwd(L, stage, ws_bytes=16) == WS
        assert bwd(L, stage, ws=A[9] + 8) == INV          # misaligned workspace
        assert bwd(L, stage, dk=A[6]) == INV              # dk == dq
        assert bwd(L, stage, dv=A[0]) == INV              # output aliases q
        assert bwd(L, stage, ws=A[8]) == INV              # workspace overlaps dv
        assert bwd(L, stage, scale=float("-inf")) == INV
    assert bwd(L, 4) == INV and bwd(L, -1) == INV
    for stage in (None, 0, 1, 2, 3):
        assert bwd(L, stage, ex=True, dtype=3) == UNS
        assert bwd(L, stage, ex=True, dtype=-1) == UNS      # only attn_bwd_f32 takes float32
        assert bwd(L, stage, ex=True, causal=5) == INV
        assert bwd(L, stage, ex=True, kv_len=A[10] + 1) == INV
        assert bwd(L, stage, ex=True, kv_len=A[7]) == INV     # kv_len inside dk
        assert bwd(L, stage, ex=True, kv_len=A[9] + 8) == INV  # kv_len inside the workspace


def test_noalloc_backward_rejections(L):
    """attn_bwd_ex_noalloc runs attn_bwd_ex's checks (no workspace argument) and refuses shapes whose workspace
    exceeds its 16 MiB array, before any HIP call."""
    INV, UNS, WS = L.ATTN_ERR_INVALID_ARG, L.ATTN_ERR_UNSUPPORTED, L.ATTN_ERR_WORKSPACE

    def na(dtype=0, layout=0, causal=0, kv_len=None, **kw):
        a = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], do=A[5], dq=A[6], dk=A[7], dv=A[8], B=1, H=1, N=8, d=64,
                 scale=0.125)
        a.update(kw)
        return L.lib.attn_bwd_ex_noalloc(dtype, layout, a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                         a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"], causal, kv_len,
                                         None)
    assert na(dq=None) == INV and na(do=A[5] + 4) == INV and na(dk=A[6]) == INV and na(dv=A[0]) == INV
    assert na(d=80) == UNS and na(dtype=2) == UNS and na(dtype=-1) == UNS and na(layout=5) == UNS
    assert na(causal=3) == INV and na(kv_len=A[7]) == INV and na(scale=float("nan")) == INV
    # 8 bytes of workspace per row: 2^21 rows fill the 16 MiB array exactly, one more 64-row block does not.
    assert L.attn_bwd_workspace_bytes(8, 16, 16384, 64) == 16 << 20
    assert na(B=8, H=16, N=16384 + 64, d=64) == WS and na(B=1, H=1, N=3_000_000, d=32) == WS


def test_f32_backward_rejections(L):
    """attn_bwd_f32 checks float32 extents: an output 8 bytes into a 2-byte-element extent still overlaps."""
    INV, UNS, WS = L.ATTN_ERR_INVALID_ARG, L.ATTN_ERR_UNSUPPORTED, L.ATTN_ERR_WORKSPACE

    def b32(**kw):
        a = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], do=A[5], dq=A[6], dk=A[7], dv=A[8], B=1, H=1, N=8, d=64,
                 scale=0.125, ws=A[9])
        a.update(kw)
        n = L.attn_bwd_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
        return L.lib.attn_bwd_f32(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                  a["B"], a["H"], a["N"], a["d"], a["scale"], a["ws"], n, None)
    assert b32(q=None) == INV and b32(d=80) == UNS and b32(ws=None) == WS
    # the fp32 forward's grid (one workgroup per 8 rows) must stay below 2^30 workgroups
    assert fwd32(L, B=1 << 14, H=1 << 10, N=1 << 10, d=32) == UNS
    assert b32(dq=A[0] + 8 * 64 * 2) == INV      # inside q's float32 extent (8 x 64 x 4 bytes), past a 2-byte one
    assert b32(dk=A[6]) == INV


def test_projection_rejections(L):
    """Every call here fails validation before a launch: bad dtype, sizes, alignment, widths, overlaps."""
    INV, UNS = L.ATTN_ERR_INVALID_ARG, L.ATTN_ERR_UNSUPPORTED

    def pf(dtype=0, x=A[0], w=A[1], y=A[2], B=2, N=5, D=64, H=2, d=32):
        return L.lib.attn_qkv_proj(dtype, x, w, y, B, N, D, H, d, None)

    def pb(dtype=0, x=A[0], w=A[1], g=A[2], dx=A[3], dw=A[4], B=2, N=5, D=64, H=2, d=32, ws=None, ws_bytes=0):
        return L.lib.attn_qkv_proj_bwd(dtype, x, w, g, dx, dw, B, N, D, H, d, ws, ws_bytes, None)

    for f in (pf, pb):
        assert f(dtype=2) == UNS and f(dtype=-1) == UNS
        assert f(B=0) == INV and f(N=-1) == INV and f(D=0) == INV and f(H=0) == INV and f(d=0) == INV
        assert f(D=60) == UNS                               # rows of x not a multiple of 16 bytes
        assert f(H=1, d=4) == UNS                           # H d_k not a multiple of 8
        assert f(B=1 << 15, N=1 << 15) == UNS               # 2^30 tokens
        assert f(x=None) == INV and f(w=A[1] + 8) == INV
    assert pf(y=A[0]) == INV and pf(y=A[1] + 16) == INV     # qkv on x / inside w
    assert pb(dx=A[4]) == INV                               # dx == dw
    assert pb(dw=A[2] + 32) == INV and pb(dx=A[0]) == INV   # outputs on inputs
    assert pb(dx=None) == INV and pb(dw=A[4] + 4) == INV
    # A shape whose products split their contraction (ViT-B/16 block) needs a workspace.
    big = dict(B=32, N=196, D=768, H=12, d=64)
    need = L.attn_qkv_proj_bwd_workspace_bytes(32, 196, 768, 12, 64)
    assert need > 0 and L.attn_qkv_proj_bwd_workspace_bytes(2, 5, 64, 2, 32) == 0
    assert L.attn_qkv_proj_bwd_workspace_bytes(2, 5, 60, 2, 32) == 0     # rejected shape
    assert pb(**big) == L.ATTN_ERR_WORKSPACE
    assert pb(ws=A[5], ws_bytes=need - 1, **big) == L.ATTN_ERR_WORKSPACE
    assert pb(ws=A[5] + 16, ws_bytes=need, **big) == INV                # not 256-byte aligned
    assert pb(ws=A[3], ws_bytes=need, **big) == INV                     # workspace on dx


def test_projection_workspace_follows_the_split_rule(L):
    """Split products write float32 partial slices: the workspace is the larger of the two products' S * M * N * 4.
    A product with at least 256 rows and columns but fewer than 192 tiles of 256 x 256 splits its contraction
    min(256 // tiles, K // 512) ways (rounded to whole 64-steps), unless it has at least 192 tiles of 128 x 128 and
    a contraction of at most 4096 (then it runs those tiles unsplit); everything else needs none."""
    def ws(B, N, D, H, d):
        return L.attn_qkv_proj_bwd_workspace_bytes(B, N, D, H, d)
    # ViT-B/16 block: dx (6272 x 768, K 2304) has 25 x 3 = 75 big tiles but 49 x 6 = 294 of 128 x 128 -> unsplit;
    # dw (768 x 2304, K 6272) has 3 x 9 = 27 big tiles (6 x 18 = 108 small ones) -> 9 splits (kchunk 704).
    assert ws(32, 196, 768, 12, 64) == 9 * 768 * 2304 * 4
    # 8 x 300 tokens, D 512, F 768: dx 10 x 2 = 20 tiles, K 768 -> 1 split; dw 2 x 3 = 6 tiles, K 2400 -> 4 splits.
    assert ws(8, 300, 512, 4, 64) == 4 * 512 * 768 * 4
    # 300 tokens, D 1024, F 1536: dx 2 x 4 = 8 tiles, K 1536 -> 3 splits; dw's K of 300 tokens is too short to split.
    assert ws(1, 300, 1024, 4, 128) == 3 * 300 * 1024 * 4
    # Under 256 rows or columns: the small-tile kernels, no workspace.
    assert ws(2, 37, 64, 1, 32) == 0 and ws(5, 7, 136, 3, 64) == 0


def test_fusion_rule(L):
    """dK/dV and dQ share a launch only for d_k <= 64 and small grids; rejected shapes answer 0."""
    assert L.attn_bwd_fused(32, 12, 196, 64) and L.attn_bwd_fused(4, 12, 2048, 64)
    assert not L.attn_bwd_fused(8, 16, 4096, 64)      # 4096 dK/dV workgroups
    assert L.attn_bwd_fused(4, 16, 2048, 64) and not L.attn_bwd_fused(6, 16, 2048, 64)  # 1024 yes, 1536 no
    assert not L.attn_bwd_fused(2, 16, 8192, 64)      # 2048 dK/dV workgroups
    assert not L.attn_bwd_fused(32, 12, 196, 128) and not L.attn_bwd_fused(1, 1, 100, 64)  # d_k 128; grid of 1
    assert not L.attn_bwd_fused(0, 12, 196, 64) and not L.attn_bwd_fused(32, 12, 196, 80)


def test_workspace_size(L):
    assert L.attn_bwd_workspace_bytes(8, 16, 4096, 64) == 2 * 8 * 16 * 4096 * 4
    assert L.attn_bwd_workspace_bytes(1, 1, 1, 64) == 512
    assert L.attn_bwd_workspace_bytes(1, 3, 100, 128) == 2560
    assert L.attn_bwd_workspace_bytes(1, 1, 8, 80) == 0
    assert L.attn_bwd_workspace_bytes(1, 1, 8, 96) == 512
    assert L.attn_bwd_workspace_bytes(0, 1, 8, 64) == 0


def test_binding_has_no_cpu_path():
    """The binding module contains no compute: it only marshals arguments into libattn.so."""
    src = open(os.path.join(ROOT, "tiled_attention_08_amd", "_lib.py")).read()
    for banned in ("oracle", "softmax", "matmul", "einsum", " @ ", "torch.exp"):
        assert banned not in src, banned


def test_c99_caller(tmp_path, L):
    """The header is plain C99 (gcc -std=c99 -Wall -Werror) and a C program linked against libattn.so gets every
    rejection from the validation layer (tests/c/abi_check.c)."""
    import shutil
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(L.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", libdir, "-lattn",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "all checks passed" in r.stdout


def test_binding_refuses_host_tensors(L, monkeypatch):
    """Every wrapper checks that its tensor arguments are GPU tensors before it reaches the C ABI: a host pointer
    handed to a kernel would fault the GPU. Host tensors here raise ValueError, and the library is never called."""
    import torch

    class NoLib:
        def __getattr__(self, name):
            raise AssertionError(f"libattn.{name} reached with a host tensor")

    monkeypatch.setattr(L, "lib", NoLib())
    B, H, N, d = 1, 2, 8, 64
    t = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    lse = torch.zeros((B, H, N), dtype=torch.float32)
    ws = torch.zeros(4096, dtype=torch.uint8)
    f32 = torch.zeros((B, H, N, d), dtype=torch.float32)
    x = torch.zeros((B, N, 128), dtype=torch.bfloat16)
    w = torch.zeros((128, 3, H, d), dtype=torch.bfloat16)
    qkv = torch.zeros((B, N, 3, H, d), dtype=torch.bfloat16)
    calls = [
        lambda: L.attn_fwd(t, t, t, t, lse, 0.125),
        lambda: L.attn_fwd_ex(t, t, t, t, lse, 0.125, causal=True),
        lambda: L.attn_fwd_f32(f32, f32, f32, f32, lse, 0.125),
        lambda: L.attn_bwd(t, t, t, t, lse, t, t, t, t, 0.125, ws),
        lambda: L.attn_bwd_f32(f32, f32, f32, f32, lse, f32, f32, f32, f32, 0.125, ws),
        lambda: L.attn_bwd_ex(t, t, t, t, lse, t, t, t, t, 0.125, ws),
        lambda: L.attn_bwd_stage(1, t, t, t, t, lse, t, t, t, t, 0.125, ws),
        lambda: L.attn_bwd_ex_noalloc(t, t, t, t, lse, t, t, t, t, 0.125),
        lambda: L.attn_qkv_proj(x, w, qkv),
        lambda: L.attn_qkv_proj_bwd(x, w, qkv, x, w, None),
        lambda: L.forward(t, t, t, 0.125),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU tensors"):
            call()


def test_ceiling_library_exports_its_header():
    """libattn_ceiling.so (the instruction-mix probe) exports what include/attn_ceiling.h declares, the binding
    lists the same names, and the mixes it names match the header's enum."""
    from tiled_attention_08_amd import ceiling
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "attn_ceiling.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))
    assert declared == sorted(ceiling.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", ceiling.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert set(declared) <= set(re.findall(r"\bT (attn_\w+)", out))
    enum = dict((k.lower(), int(v)) for k, v in re.findall(r"ATTN_MIX_(\w+)\s*=\s*(\d+)", text))
    assert enum == {k: v[0] for k, v in ceiling.MIXES.items()}
    L = ceiling.load()
    assert L.attn_mix_ceiling_workspace_bytes() > 0
    assert L.attn_mix_ceiling_flop(10) == 256 * 8 * 10 * 8 * 32768.0
    # Rejected on the host before any HIP call: unknown mix, bad iteration count, null workspace.
    import ctypes
    ms = ctypes.c_float()
    big = L.attn_mix_ceiling_workspace_bytes()
    assert L.attn_mix_ceiling(9, 10, 0x1000, big, ctypes.byref(ms), None) == -1
    assert L.attn_mix_ceiling(1, 0, 0x1000, big, ctypes.byref(ms), None) == -1
    assert L.attn_mix_ceiling(1, 10, None, big, ctypes.byref(ms), None) == -1
    assert L.attn_mix_ceiling(1, 10, 0x1000, 16, ctypes.byref(ms), None) == -3
