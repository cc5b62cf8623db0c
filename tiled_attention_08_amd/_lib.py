"""ctypes binding of libattn.so: the same entry points as include/attn.h, taking torch tensors.

Argument marshalling only: shapes and dtypes are read off the tensors, their
device pointers and the stream handle are passed to the C ABI, and a non-zero
status becomes an ``AttnError``. Every step of the computation runs in the HIP
kernels; there is no fallback. Importing this module raises ImportError if the
library has not been built (``python -m tiled_attention_08_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4
ATTN_DTYPE_BF16 = 0
ATTN_DTYPE_F16 = 1
LAYOUTS = {"bhnd": 0, "bnhd": 1, "qkv_packed": 2}

# Every symbol include/attn.h declares.
EXPORTS = ("attn_fwd", "attn_fwd_f32", "attn_fwd_ex", "attn_bwd", "attn_bwd_f32", "attn_bwd_ex", "attn_bwd_stage",
           "attn_bwd_ex_noalloc", "attn_bwd_fused", "attn_bwd_workspace_bytes", "attn_qkv_proj", "attn_qkv_proj_bwd",
           "attn_qkv_proj_bwd_workspace_bytes", "attn_status_string")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tiled_attention_08_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp]
    lib.attn_fwd_f32.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_f32.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    lib.attn_bwd_f32.restype = i
    lib.attn_fwd_ex.argtypes = [i, i, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.attn_fwd_ex.restype = i
    lib.attn_bwd_ex.argtypes = [i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.attn_bwd_ex.restype = i
    lib.attn_bwd_stage.argtypes = [i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.attn_bwd_stage.restype = i
    lib.attn_bwd_ex_noalloc.argtypes = [i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.attn_bwd_ex_noalloc.restype = i
    lib.attn_bwd_fused.argtypes = [i, i, i, i]
    lib.attn_bwd_fused.restype = i
    lib.attn_qkv_proj.argtypes = [i, vp, vp, vp, i, i, i, i, i, vp]
    lib.attn_qkv_proj.restype = i
    lib.attn_qkv_proj_bwd.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    lib.attn_qkv_proj_bwd.restype = i
    lib.attn_qkv_proj_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_qkv_proj_bwd_workspace_bytes.restype = sz
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libattn status {status}: {attn_status_string(status)}")


def attn_status_string(status: int) -> str:
    return lib.attn_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on_gpu(*ts) -> None:
    """Every tensor argument must be in GPU memory, all on one device (a host pointer reaching a kernel would fault
    the GPU). Checked before anything is launched; None (an absent optional buffer) is skipped."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"tensor arguments must be GPU tensors (got one on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensor arguments must share one device ({t.device} vs {dev})")


def _shape(q, *others):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d_k]")
    for t in others:
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"shape mismatch: {tuple(t.shape)} vs {tuple(q.shape)}")
    for t in (q,) + others:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d_k]")
        if t.dtype != q.dtype:
            raise ValueError("all tensors must share one dtype")
    return tuple(int(x) for x in q.shape)


def _dims(layout: str, qkv, others=()):
    """(B, H, N, d) from tensors in ``layout``; checks every row is contiguous and each tensor has its layout's strides.

    qkv: the q, k, v (or dq, dk, dv) tensors; others: o / dO. In "bhnd" all are [B, H, N, d] contiguous; in
    "bnhd" all are [B, N, H, d] contiguous; in "qkv_packed" q, k, v are the [B, N, H, d] slices 0, 1, 2 of one
    [B, N, 3, H, d] tensor and the others [B, N, H, d] contiguous.
    """
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    t0 = qkv[0]
    if t0.dim() != 4:
        raise ValueError("tensors must be 4-D")
    if layout == "bhnd":
        B, H, N, d = (int(x) for x in t0.shape)
    else:
        B, N, H, d = (int(x) for x in t0.shape)
    for t in tuple(qkv) + tuple(others):
        if tuple(t.shape) != tuple(t0.shape) or t.dtype != t0.dtype:
            raise ValueError("all tensors must share one shape and dtype")
    for t in others:
        if not t.is_contiguous():
            raise ValueError("o / dO must be contiguous")
    if layout == "qkv_packed":
        want = (N * 3 * H * d, 3 * H * d, d, 1)
        for t in qkv:
            if tuple(t.stride()) != want:
                raise ValueError("qkv_packed: q, k, v must be slices [:, :, 0/1/2] of one contiguous [B, N, 3, H, d]")
    else:
        for t in qkv:
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
    return B, H, N, d


def _check_lse(lse, B, H, N):
    import torch
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float16:
        return ATTN_DTYPE_F16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _check_kv_len(kv_len, B):
    import torch
    if kv_len is None:
        return
    if kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,) or not kv_len.is_contiguous() or not kv_len.is_cuda:
        raise ValueError("kv_len must be a contiguous int32 device tensor of shape [B]")


def attn_fwd(q, k, v, o, lse, scale: float, stream=None) -> None:
    """bf16 forward into caller-provided ``o`` (bf16 [B,H,N,d]) and ``lse`` (float32 [B,H,N])."""
    import torch
    _on_gpu(q, k, v, o, lse)
    B, H, N, d = _shape(q, k, v, o)
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_fwd takes bfloat16 tensors")
    _check_lse(lse, B, H, N)
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale), _stream(stream)))


def attn_fwd_ex(q, k, v, o, lse, scale: float, causal: bool = False, kv_len=None, stream=None,
                layout: str = "bhnd") -> None:
    """Forward with masks and layouts: ``causal`` (query i sees keys j <= i), ``kv_len`` (int32 [B] device tensor
    of valid keys), ``layout`` "bhnd", "bnhd" or "qkv_packed" (see ``_dims``)."""
    _on_gpu(q, k, v, o, lse, kv_len)
    B, H, N, d = _dims(layout, (q, k, v), (o,))
    _check_lse(lse, B, H, N)
    _check_kv_len(kv_len, B)
    _check(lib.attn_fwd_ex(_dtype_code(q), LAYOUTS[layout], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N,
                           d, float(scale), int(bool(causal)), _ptr(kv_len), _stream(stream)))


def attn_fwd_f32(q, k, v, o, lse, scale: float, stream=None) -> None:
    """float32 forward into caller-provided ``o`` (float32 [B,H,N,d]) and ``lse``."""
    import torch
    _on_gpu(q, k, v, o, lse)
    B, H, N, d = _shape(q, k, v, o)
    if q.dtype != torch.float32:
        raise ValueError("attn_fwd_f32 takes float32 tensors")
    _check_lse(lse, B, H, N)
    _check(lib.attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                            _stream(stream)))


def attn_bwd_fused(B: int, H: int, N: int, d_k: int) -> bool:
    """Whether the backward of this shape runs its dK/dV and dQ work as one launch (stage 3)."""
    return bool(lib.attn_bwd_fused(B, H, N, d_k))


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d_k: int) -> int:
    return int(lib.attn_bwd_workspace_bytes(B, H, N, d_k))


def attn_bwd(q, k, v, o, lse, do, dq, dk, dv, scale: float, workspace, stream=None) -> None:
    """bf16 backward into caller-provided ``dq``, ``dk``, ``dv``; ``workspace`` is a uint8 device tensor."""
    import torch
    _on_gpu(q, k, v, o, lse, do, dq, dk, dv, workspace)
    B, H, N, d = _shape(q, k, v, o, do, dq, dk, dv)
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_bwd takes bfloat16 tensors")
    _check_lse(lse, B, H, N)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, H, N, d, float(scale), _ptr(workspace), ws_bytes, _stream(stream)))


def attn_bwd_f32(q, k, v, o, lse, do, dq, dk, dv, scale: float, workspace, stream=None) -> None:
    """float32 backward into caller-provided ``dq``, ``dk``, ``dv`` (float32 [B,H,N,d])."""
    import torch
    _on_gpu(q, k, v, o, lse, do, dq, dk, dv, workspace)
    B, H, N, d = _shape(q, k, v, o, do, dq, dk, dv)
    if q.dtype != torch.float32:
        raise ValueError("attn_bwd_f32 takes float32 tensors")
    _check_lse(lse, B, H, N)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                            B, H, N, d, float(scale), _ptr(workspace), ws_bytes, _stream(stream)))


def attn_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, scale: float, workspace, causal: bool = False, kv_len=None,
                stream=None, layout: str = "bhnd") -> None:
    """Backward with the masks and layout of attn_fwd_ex (which must match the forward's)."""
    _on_gpu(q, k, v, o, lse, do, dq, dk, dv, kv_len, workspace)
    B, H, N, d = _dims(layout, (q, k, v), (o, do))
    _dims(layout, (dq, dk, dv))
    _check_lse(lse, B, H, N)
    _check_kv_len(kv_len, B)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_bwd_ex(_dtype_code(q), LAYOUTS[layout], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                           _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(kv_len),
                           _ptr(workspace), ws_bytes, _stream(stream)))


def attn_bwd_ex_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool = False, kv_len=None,
                        stream=None, layout: str = "bhnd") -> None:
    """attn_bwd_ex with the library's own device workspace (16 MiB per GPU): for callers that cannot allocate.
    Calls that overlap in time on one GPU race on that workspace."""
    _on_gpu(q, k, v, o, lse, do, dq, dk, dv, kv_len)
    B, H, N, d = _dims(layout, (q, k, v), (o, do))
    _dims(layout, (dq, dk, dv))
    _check_lse(lse, B, H, N)
    _check_kv_len(kv_len, B)
    _check(lib.attn_bwd_ex_noalloc(_dtype_code(q), LAYOUTS[layout], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                   int(bool(causal)), _ptr(kv_len), _stream(stream)))


def attn_bwd_stage(stage: int, q, k, v, o, lse, do, dq, dk, dv, scale: float, workspace, causal: bool = False,
                   kv_len=None, stream=None, layout: str = "bhnd") -> None:
    """One stage (0 prep, 1 dK/dV, 2 dQ, 3 = 1 and 2 as attn_bwd_ex runs them) of attn_bwd_ex; same arguments."""
    _on_gpu(q, k, v, o, lse, do, dq, dk, dv, kv_len, workspace)
    B, H, N, d = _dims(layout, (q, k, v), (o, do))
    _dims(layout, (dq, dk, dv))
    _check_lse(lse, B, H, N)
    _check_kv_len(kv_len, B)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_bwd_stage(int(stage), _dtype_code(q), LAYOUTS[layout], _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                              int(bool(causal)), _ptr(kv_len), _ptr(workspace), ws_bytes, _stream(stream)))


def _proj_dims(x, w):
    """(B, N, D, H, d) of a projection: x [B, N, D], w [D, 3, H, d], both contiguous, one 16-bit dtype."""
    if x.dim() != 3 or w.dim() != 4 or int(w.shape[0]) != int(x.shape[2]) or int(w.shape[1]) != 3:
        raise ValueError("x must be [B, N, D] and w [D, 3, H, d_k]")
    if not x.is_contiguous() or not w.is_contiguous() or x.dtype != w.dtype:
        raise ValueError("x and w must be contiguous and share one dtype")
    B, N, D = (int(a) for a in x.shape)
    return B, N, D, int(w.shape[2]), int(w.shape[3])


def _check_packed(t, B, N, H, d, dtype, what):
    if tuple(t.shape) != (B, N, 3, H, d) or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{what} must be a contiguous [B, N, 3, H, d_k] tensor of the inputs' dtype")


def attn_qkv_proj(x, w, qkv, stream=None) -> None:
    """qkv[b, n, t, h, :] = sum over c of x[b, n, c] w[c, t, h, :] (t = 0, 1, 2: Q, K, V)."""
    _on_gpu(x, w, qkv)
    B, N, D, H, d = _proj_dims(x, w)
    _check_packed(qkv, B, N, H, d, x.dtype, "qkv")
    _check(lib.attn_qkv_proj(_dtype_code(x), _ptr(x), _ptr(w), _ptr(qkv), B, N, D, H, d, _stream(stream)))


def attn_qkv_proj_bwd_workspace_bytes(B: int, N: int, D: int, H: int, d_k: int) -> int:
    return int(lib.attn_qkv_proj_bwd_workspace_bytes(B, N, D, H, d_k))


def attn_qkv_proj_bwd(x, w, dqkv, dx, dw, workspace, stream=None) -> None:
    """dx = dqkv W^T per token; dw = X^T dqkv over all tokens. ``workspace``: a device buffer of at least
    attn_qkv_proj_bwd_workspace_bytes(...) bytes (None when that is 0)."""
    _on_gpu(x, w, dqkv, dx, dw, workspace)
    B, N, D, H, d = _proj_dims(x, w)
    _check_packed(dqkv, B, N, H, d, x.dtype, "dqkv")
    if tuple(dx.shape) != tuple(x.shape) or tuple(dw.shape) != tuple(w.shape):
        raise ValueError("dx / dw must have the shapes of x / w")
    for t in (dx, dw):
        if not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError("dx / dw must be contiguous tensors of the inputs' dtype")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.attn_qkv_proj_bwd(_dtype_code(x), _ptr(x), _ptr(w), _ptr(dqkv), _ptr(dx), _ptr(dw), B, N, D, H, d,
                                 _ptr(workspace), nbytes, _stream(stream)))


# ---------------------------------------------------------------- allocating conveniences

def forward(q, k, v, scale: float, stream=None, causal: bool = False, kv_len=None):
    """Allocate O and lse with torch, then run the forward matching q's dtype (bf16, float16 or float32)."""
    import torch
    B, H, N, d = _shape(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if q.dtype == torch.float32:
        if causal or kv_len is not None:
            raise ValueError("the float32 forward takes no mask")
        attn_fwd_f32(q, k, v, o, lse, scale, stream)
    elif q.dtype == torch.bfloat16 and not causal and kv_len is None:
        attn_fwd(q, k, v, o, lse, scale, stream)
    else:
        attn_fwd_ex(q, k, v, o, lse, scale, causal=causal, kv_len=kv_len, stream=stream)
    return o, lse


def workspace_for(q) -> "torch.Tensor":
    import torch
    B, H, N, d = (int(x) for x in q.shape)
    return torch.empty(attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)


def backward(q, k, v, o, lse, do, scale: float, workspace=None, stream=None, causal: bool = False, kv_len=None):
    """Allocate dQ, dK, dV (and the workspace unless given), then run the backward matching q's dtype."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = workspace_for(q)
    if q.dtype == torch.float32:
        if causal or kv_len is not None:
            raise ValueError("the float32 backward takes no mask")
        attn_bwd_f32(q, k, v, o, lse, do, dq, dk, dv, scale, workspace, stream)
    elif q.dtype == torch.bfloat16 and not causal and kv_len is None:
        attn_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, workspace, stream)
    else:
        attn_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, scale, workspace, causal=causal, kv_len=kv_len, stream=stream)
    return dq, dk, dv


def qkv_proj(x, w, stream=None):
    """Allocate the packed [B, N, 3, H, d_k] output and project; returns (qkv, q, k, v), where q, k, v are the
    [B, N, H, d_k] slices that attn_fwd_ex / attn_bwd_ex take with layout="qkv_packed"."""
    import torch
    B, N, D, H, d = _proj_dims(x, w)
    qkv = torch.empty((B, N, 3, H, d), dtype=x.dtype, device=x.device)
    attn_qkv_proj(x, w, qkv, stream)
    return qkv, qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]


def proj_workspace_for(x, w):
    """A workspace for attn_qkv_proj_bwd with these inputs (None when the shape needs none)."""
    import torch
    B, N, D, H, d = _proj_dims(x, w)
    n = attn_qkv_proj_bwd_workspace_bytes(B, N, D, H, d)
    return torch.empty(n, dtype=torch.uint8, device=x.device) if n else None


def qkv_proj_bwd(x, w, dqkv, workspace=None, stream=None):
    """Allocate dx and dw (and the workspace unless given), then run the projection's backward; returns (dx, dw)."""
    import torch
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    if workspace is None:
        workspace = proj_workspace_for(x, w)
    attn_qkv_proj_bwd(x, w, dqkv, dx, dw, workspace, stream)
    return dx, dw
