"""Build the gfx950 attention library (libfa2.so) in-tree with hipcc.

    python -m exact_attention_11_amd.build

The library exports the C ABI of include/fa2.h.  It links the HIP runtime by its
SONAME (libamdhip64.so.7); loaded after ``import torch`` it binds to the runtime
torch already mapped, so torch's streams and memory are valid inside it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa2.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_command(out: str = LIB_PATH) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # Keep packed fp32 (v_pk_*_f32) instructions out of the generated code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
        os.path.join(CSRC, "fa2_api.hip"),
        "-o", out,
    ]


def build(out: str = LIB_PATH, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with code {res.returncode}")
    # MFMAs and LDS copies written as inline assembly are invisible to the
    # compiler's hazard recognizer: check their spacing on the built code before
    # installing it.
    from . import hazards
    bad = hazards.check_library(tmp)
    if bad:
        os.remove(tmp)
        raise RuntimeError("hazards in the built kernels (function, kind, first address, second address, "
                           f"wait states): {bad[:8]}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
