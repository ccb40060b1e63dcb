"""Build libdecode_attn.so for gfx950 with hipcc, in-tree.

    python -m decode_phase_attention_paged_amd.build

The library links the HIP runtime by soname (libamdhip64.so.7). Loaded after
``import torch`` it binds to the runtime torch already mapped, so torch's
hipStream_t handles are valid inside it.
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
LIB_NAME = "libdecode_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["kernels.hip", "append.hip", "prefill.hip", "api.cpp"]
ARCH = "gfx950"

# Packed-FP32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build")
    return path


def compile_cmd(out: str = LIB_PATH, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-mcode-object-version=5", "-Wall", "-Wno-unused-command-line-argument",
        *DEVICE_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *extra,
        *[os.path.join(CSRC, s) for s in SOURCES], "-o", out,
    ]


def build(verbose: bool = True) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature name; that warning is
        # expected. Anything else is shown.
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if any(ln.strip() for ln in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
