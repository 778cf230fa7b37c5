"""Build libslt.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each translation unit compiles to an object in parallel, then one shared
library is linked next to this file.  Run as a module or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libslt.so")
SOURCES = ["rowops.hip", "gemm.hip", "attention.hip", "flash.hip", "decode.hip", "api.hip", "calib.hip", "noalloc.hip"]
ARCH = os.environ.get("SLT_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            # keep packed-fp32 instructions out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str, defines=()) -> None:
    cmd = [_hipcc(), *flags(), *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)


def build(verbose: bool = True, defines=(), out: str = LIB) -> str:
    """Compile every source and link ``out``.  ``defines`` are extra -D
    macros (kernel tuning constants; the defaults are the tuned values)."""
    objdir = os.path.join(HERE, "_build", "_".join(defines) if defines else "default")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], defines), zip(SOURCES, objs)))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
