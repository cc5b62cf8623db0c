"""Build libattn.so (the HIP kernels and the C ABI) and libattn_ceiling.so (the instruction-mix probe that
measured roofline fractions are read against) in-tree for gfx950.

    python -m tiled_attention_08_amd.build          # compile
    python -m tiled_attention_08_amd.build --asm    # also keep the gfx950 assembly under _build/asm

Always recompiles; the results land next to this file.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
CEILING_LIB = os.path.join(PKG, "libattn_ceiling.so")
CEILING_SRC = "mix_ceiling.hip"
SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_proj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # Packed fp32 VALU ops stay off: only scalar fp32 VALU code is generated.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False, asm: bool = False) -> str:
    """Compile every source into ``libattn.so``; return its path. Raises on failure."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append(([cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj], obj))
        if asm:
            asmdir = os.path.join(ROOT, "_build", "asm")
            os.makedirs(asmdir, exist_ok=True)
            jobs.append(([cc, *flags(), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o",
                          os.path.join(asmdir, src.replace(".hip", f"-{ARCH}.s"))], None))
    ceiling_obj = os.path.join(objdir, CEILING_SRC.replace(".hip", ".o"))
    jobs.append(([cc, *flags(), "-c", os.path.join(CSRC, CEILING_SRC), "-o", ceiling_obj], None))
    # The translation units are independent: compile them side by side.
    procs = []
    for cmd, _ in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
    failed = [" ".join(cmd) for (cmd, _), p in zip(jobs, procs) if p.wait() != 0]
    if failed:
        raise RuntimeError("compilation failed: " + "; ".join(failed))
    objs = [obj for _, obj in jobs if obj is not None]
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = CEILING_LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", ceiling_obj, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, CEILING_LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--asm", action="store_true", help="also write gfx950 assembly to _build/asm")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(verbose=a.verbose, asm=a.asm)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
