"""Build libdecode_attn.so for gfx950 with hipcc, in-tree.

    python -m decode_phase_attention_paged_amd.build

The library links the HIP runtime by soname (libamdhip64.so.7). Loaded after
``import torch`` it binds to the runtime torch already mapped, so torch's
hipStream_t handles are valid inside it.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdecode_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["kernels.hip", "append.hip", "prefill.hip", "hbm_reference.hip", "api.cpp"]
ARCH = "gfx950"

# Packed-FP32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build")
    return path


def _common_flags(extra=()) -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-mcode-object-version=5", "-Wall", "-Wno-unused-command-line-argument",
        *DEVICE_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *extra,
    ]


def compile_cmd(out: str = LIB_PATH, extra=()) -> list:
    """One hipcc line that compiles and links every source (for reference and tools)."""
    return [hipcc(), *_common_flags(extra), "-shared",
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def _filter_stderr(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is
    # expected, and the kernel resource remarks are read by scratch_use(). Anything else is
    # shown.
    lines = [ln for ln in text.splitlines()
             if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln]
    return "\n".join(lines) + "\n" if any(ln.strip() for ln in lines) else ""


# Every kernel is built to keep its live values in registers: a build that spills to
# scratch memory runs several times slower, so the build fails if any kernel reports
# scratch. The compiler's resource remarks name each kernel and its scratch bytes per lane.
RESOURCE_FLAGS = ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]


def scratch_use(remarks: str) -> dict:
    """{kernel symbol: scratch bytes per lane} from the compiler's resource remarks."""
    use, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None:
            use[name] = int(m.group(1))
    return use


def build(verbose: bool = True) -> str:
    """Compile the library (always recompiles) and return its path. The sources compile
    to objects in parallel (one hipcc per file), then link into one shared library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = tempfile.mkdtemp(prefix="decode_attn_build_")
    try:
        def compile_one(src):
            obj = os.path.join(objdir, src + ".o")
            cmd = [hipcc(), *_common_flags(RESOURCE_FLAGS), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            results = list(pool.map(compile_one, SOURCES))
        spilled = []
        for (obj, res), src in zip(results, SOURCES):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed on {src} with exit code {res.returncode}")
            if verbose and _filter_stderr(res.stderr).strip():
                sys.stderr.write(_filter_stderr(res.stderr))
            use = scratch_use(res.stderr)
            if src.endswith(".hip") and not use:
                raise RuntimeError(f"no kernel resource remarks from {src}; cannot check scratch")
            spilled += [f"{src}: {k} ({v} bytes/lane)" for k, v in use.items() if v > 0]
        if spilled:
            raise RuntimeError("kernels spill to scratch memory:\n  " + "\n  ".join(spilled))
        tmp = LIB_PATH + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
               *[obj for obj, _ in results], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    build()
