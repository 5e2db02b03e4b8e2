"""The host-side code under AddressSanitizer and UBSan, with the library's
debug plan checks (CPU only, no GPU, no HIP call):

  * the library is built with its host code instrumented (the device code is
    compiled as always) and -DGLA_DEBUG, which checks the plan and workspace
    arithmetic as the planners make it;
  * tests/c/plan_check.cpp compiles the host dispatch into a checker that
    replays the device planner on the host and checks item tiling, slot
    indices, workspace regions and the workgroup mapping for the long-context,
    packed (the seeded 32-sequence workload included) and ragged plans;
  * the plain C program of tests/c/abi_from_c.c runs against that build;
  * tests/test_abi.py runs in a process with the sanitizer runtime preloaded,
    against that build;
  * the oracle (oracle/gla_oracle.c), built with gcc's sanitizers, runs its
    pin tests.
Any sanitizer report aborts the process that made it (no recovery)."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_gated_recurrent_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "tests", "_build", "host_sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["gla_kernels.hip", "gla_fwd_mfma.hip", "gla_bwd_mfma.hip", "gla_bwd_valu.hip",
           "gla_bwd_wide.hip", "gla_conv.hip", "gla_api.cpp"]
# host-only instrumentation: every sanitizer flag applies to the host side
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HIP_FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
             "-DGLA_DEBUG", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC] + HOST_SAN
LINK_SAN = ["-fsanitize=address,undefined", "-shared-libasan"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which("gcc") is None,
                                reason="needs ROCm's clang and gcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    return r.returncode, out


def _torch_lib():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def _clang_asan_runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    assert rt, "clang's AddressSanitizer runtime not found"
    return rt[-1]


@pytest.fixture(scope="module")
def hsan():
    """Objects, the instrumented library and the two host programs."""
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
        rc, out = _run([CLANG] + HIP_FLAGS + ["-c", src, "-o", obj])
        assert rc == 0, out
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [
        os.path.join(ROOT, "tests", "c", "plan_check.cpp")]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(compile_one, srcs)))
    lib_objs = [objs[os.path.join(CSRC, s)] for s in SOURCES]
    tl = _torch_lib()
    rt = _clang_asan_runtime()
    hip = ["-L" + tl, "-l:libamdhip64.so", "-Wl,-rpath," + tl,
           "-Wl,-rpath," + os.path.dirname(rt)]
    lib = os.path.join(BUILD, "libgla_hsan.so")
    rc, out = _run([CLANG, "-shared"] + LINK_SAN + ["-o", lib] + lib_objs + hip)
    assert rc == 0, out
    # the checker compiles gla_api.cpp into itself, so it links the others
    plan_check = os.path.join(BUILD, "plan_check")
    others = [o for o in lib_objs if not o.endswith("gla_api.o")]
    rc, out = _run([CLANG] + LINK_SAN + ["-o", plan_check,
                                         objs[os.path.join(ROOT, "tests", "c", "plan_check.cpp")]]
                   + others + hip)
    assert rc == 0, out
    abi = os.path.join(BUILD, "abi_from_c")
    rc, out = _run([CLANG, "-x", "c", "-std=c99", "-pedantic", "-Wall", "-Werror", "-g"]
                   + LINK_SAN + ["-fno-sanitize-recover=all", "-I" + INCLUDE,
                                 os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-x", "none",
                                 lib, "-Wl,-rpath," + BUILD] + hip + ["-o", abi])
    assert rc == 0, out
    return {"lib": lib, "plan_check": plan_check, "abi": abi, "rt": rt}


def test_plan_arithmetic_under_sanitizers(hsan):
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS["varlen"]
    c5 = ",".join(str(int(x)) for x in W.varlen_lengths(spec["seed"], spec["N"], spec["max_len"]))
    env = dict(os.environ, **ENV_SAN)
    env.pop("GLA_TARGET_WGS", None)
    rc, out = _run([hsan["plan_check"], c5], env=env, timeout=600)
    print(out)
    assert rc == 0, out
    assert "0 failures" in out


def test_c_program_under_sanitizers(hsan):
    rc, out = _run([hsan["abi"]], env=dict(os.environ, **ENV_SAN), timeout=120)
    assert rc == 0, out
    assert out.strip().endswith("ok"), out


def test_abi_suite_under_sanitizers(hsan):
    env = dict(os.environ, **ENV_SAN)
    env["LD_PRELOAD"] = hsan["rt"]
    env["GLA_TEST_HOST_LIB"] = hsan["lib"]
    rc, out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_abi.py")], env=env, cwd=ROOT, timeout=600)
    assert rc == 0, out
    assert " passed" in out and "failed" not in out, out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    rc, out = _run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", lib,
                    os.path.join(ROOT, "oracle", "gla_oracle.c"), "-lpthread"])
    assert rc == 0, out
    rc, gcc_asan = _run(["gcc", "-print-file-name=libasan.so"])
    env = dict(os.environ, **ENV_SAN)
    env["LD_PRELOAD"] = gcc_asan.strip()
    env["GLA_ORACLE_LIB"] = lib
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle*_pins.py")))
    assert len(pins) >= 4
    rc, out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + pins,
                   env=env, cwd=ROOT, timeout=900)
    assert rc == 0, out
    assert " passed" in out and "failed" not in out, out
