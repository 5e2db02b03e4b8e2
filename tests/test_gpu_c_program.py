"""The library driven from a plain C program on the GPU (tests/c/
gla_from_c_gpu.c): device memory from the HIP runtime, no Python or torch in
its process, a chunked forward and a decode step checked against the fp64
oracle's C entry points. The program links the same HIP runtime that
libgla.so was linked against (torch/lib/libamdhip64.so)."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunked_gated_recurrent_amd")
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_runs_forward_and_decode_on_the_gpu(tmp_path):
    from chunked_gated_recurrent_amd import build as hip_build
    for lib in (os.path.join(PKG, "libgla.so"), os.path.join(ORACLE, "liboracle.so")):
        assert os.path.exists(lib), lib + " is not built"
    tlib = hip_build._torch_lib()
    exe = str(tmp_path / "gla_from_c_gpu")
    cmd = ["gcc", "-std=gnu99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "gla_from_c_gpu.c"),
           "-L", PKG, "-lgla", "-Wl,-rpath," + PKG,
           "-L", ORACLE, "-loracle", "-Wl,-rpath," + ORACLE,
           "-L", tlib, "-l:libamdhip64.so", "-Wl,-rpath," + tlib, "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok"), r.stdout
