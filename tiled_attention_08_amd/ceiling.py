"""Binding of libattn_ceiling.so (include/attn_ceiling.h): the sustained matrix-core rate of the chip for each
attention kernel's instruction mix, the ceiling a measured roofline fraction is read against. Argument
marshalling only; the probe runs on the GPU."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_ceiling.so")
EXPORTS = ("attn_mix_ceiling", "attn_mix_ceiling_flop", "attn_mix_ceiling_workspace_bytes")
# Mix names and codes (ATTN_MIX_*), with the mix per 8 products: vector-ALU instructions (exponentials among
# them) and 16-byte + 8-byte LDS reads, equal to the kernel's instruction counters per product x 8.
MIXES = {"constant": (0, "products only, constant operands"),
         "random": (1, "products only, random operands"),
         "dkdv": (2, "dK/dV kernels, d_k 64: 36 VALU (8 exp), 8 + 8 LDS reads per 8 products"),
         "dq": (3, "dQ kernel, d_k 64: 40 VALU (11 exp), 2 + 4 LDS reads per 8 products"),
         "fwd64": (4, "forward, d_k 64: 54 VALU (16 exp), 4 + 8 LDS reads per 8 products"),
         "fwd128": (5, "forward, d_k 128: 26 VALU (8 exp), 4 + 8 LDS reads per 8 products")}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tiled_attention_08_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.attn_mix_ceiling_workspace_bytes.argtypes = []
        L.attn_mix_ceiling_workspace_bytes.restype = ctypes.c_size_t
        L.attn_mix_ceiling_flop.argtypes = [ctypes.c_int]
        L.attn_mix_ceiling_flop.restype = ctypes.c_double
        L.attn_mix_ceiling.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_float), ctypes.c_void_p]
        L.attn_mix_ceiling.restype = ctypes.c_int
        _lib = L
    return _lib


def mix_ceiling(mix: str, iters: int = 20000, stream=None) -> dict:
    """Runs the probe for one mix on cuda:0 (blocking) and returns its rate in TFLOP/s."""
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("the probe needs a GPU")
    if mix not in MIXES:
        raise ValueError(f"mix must be one of {sorted(MIXES)}")
    L = load()
    nbytes = L.attn_mix_ceiling_workspace_bytes()
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ms = ctypes.c_float(0.0)
    st = (stream or torch.cuda.current_stream()).cuda_stream
    rc = L.attn_mix_ceiling(MIXES[mix][0], int(iters), ws.data_ptr(), nbytes, ctypes.byref(ms), st)
    if rc != 0:
        raise RuntimeError(f"attn_mix_ceiling({mix}) returned {rc}")
    tflops = L.attn_mix_ceiling_flop(int(iters)) / (ms.value * 1e-3) / 1e12
    return {"mix": mix, "description": MIXES[mix][1], "value": round(tflops, 1), "unit": "TFLOP/s",
            "ms": round(ms.value, 4)}
