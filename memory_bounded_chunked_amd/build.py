"""Build the HIP library ``libdit_block.so`` in-tree for gfx950.

Run ``python -m memory_bounded_chunked_amd.build``. Compiles every time it is
called. Sources: ``csrc/*.hip`` (kernels) and ``csrc/dit_block.cpp`` (C ABI
and schedule).
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdit_block.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["modnorm.hip", "gemm.hip", "attention.hip", "qk_transform.hip", "final_layer.hip", "lora.hip",
           "dit_block.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    return r


def build(verbose: bool = True) -> str:
    """Compile each source to an object in parallel, then link the shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = False
    for cmd, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            failed = True
            sys.stderr.write(out + err)
            sys.stderr.write("\nFAILED: " + " ".join(cmd) + "\n")
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB + ".tmp"
    # -z defs: a kernel whose host-side stub was not emitted fails here, not at load time
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build()
