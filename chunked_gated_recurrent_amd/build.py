"""Build the HIP library ``libgla.so`` in-tree for gfx950.

Sources (csrc/) are compiled with hipcc; the shared object is linked against
the HIP runtime that PyTorch ships (``torch/lib/libamdhip64.so``), so that a
process which has imported torch holds ONE HIP runtime and the library can
run on torch's streams. Without torch in the process the same runtime is
found through the rpath.

Usage: ``python -m chunked_gated_recurrent_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgla.so")
SOURCES = ["gla_kernels.hip", "gla_fwd_mfma.hip", "gla_bwd_mfma.hip", "gla_bwd_valu.hip",
           "gla_bwd_wide.hip", "gla_conv.hip",
           "gla_api.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _torch_lib() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is required to locate its HIP runtime")
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError("torch/lib/libamdhip64.so not found")
    return d


def compile_flags(debug: bool = False):
    f = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall",
         "-I" + INCLUDE, "-I" + CSRC,
         # keep packed-fp32 instructions out of the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    f += ["-O0", "-g"] if debug else ["-O3"]
    return f


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + compile_flags(debug) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature: harmless, drop it
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(debug: bool = False, verbose: bool = True) -> str:
    """Compile every source and link libgla.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    tlib = _torch_lib()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-shared", "-o", tmp] + objs + [
        "-L" + tlib, "-l:libamdhip64.so", "-Wl,-rpath," + tlib,
        "-Wl,--no-undefined", "-Wl,-z,defs"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(debug="--debug" in sys.argv)
