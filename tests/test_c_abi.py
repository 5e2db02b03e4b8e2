"""The C ABI from a plain C99 program (tests/c/abi_from_c.c): the header
compiles under -std=c99 -pedantic -Werror, the program links libgla.so and
runs without Python or torch in its process. It exercises only host-side
behaviour (version, status text, workspace queries, validation errors), so
it runs without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunked_gated_recurrent_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(PKG, "libgla.so")
    if not os.path.exists(lib):
        pytest.skip("libgla.so is not built")
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
           "-L", PKG, "-lgla", "-Wl,-rpath," + PKG, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok"), r.stdout
