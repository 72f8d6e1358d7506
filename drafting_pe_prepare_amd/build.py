"""Builds libpe.so (HIP for gfx950) in-tree with hipcc.

    python -m drafting_pe_prepare_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled; the
library links the HIP runtime only (every kernel is the library's own).  The
output lands next to this file, where the Python binding looks for it.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libpe.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["pe_meta.hip", "pe_norm.hip", "pe_gemm.hip", "pe_mm.hip", "pe_attn.hip", "pe_sample.hip",
           "pe_api.cpp"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", CSRC, "-I", INCLUDE]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src, flags, objdir):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc()] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj, msgs


def build(verbose: bool = True, out: str = None, objdir: str = None, defines=()) -> str:
    """Compile every source and link libpe.so (or `out`).  `defines` are
    extra -D macros for experimental variants.  Holds no global state, so
    several builds (with their own `out` and `objdir`) may run at once."""
    out = out or OUT
    objdir = objdir or OBJDIR
    flags = FLAGS + [f"-D{d}" for d in defines]
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(lambda src: _compile(src, flags, objdir), SOURCES))
    for obj, msgs in results:
        if verbose and msgs:
            print("\n".join(msgs), file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results] + \
          ["-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
