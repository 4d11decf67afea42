"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument validation, handle bookkeeping, error messages) is compiled
with g++ and both sanitizers; the kernels' objects from the regular build are
linked in unchanged (their host code is only launch glue, and nothing here
reaches a launch).  Then
  1. tests/host_asan_driver.cpp runs against that library with leak detection
     on: size queries, handle creation and destruction, and every entry point
     with one argument out of range, from several threads;
  2. the host ABI tests (test_abi_host.py) run against it in a child process.
The GPU is hidden from both processes: a call that slipped past validation
would fail to launch rather than touch device memory."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "test_activation_aware_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include")),
                                reason="needs g++ and the ROCm headers")


def _env(**extra):
    env = dict(os.environ)
    env.update(HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(extra)
    return env


def _run(cmd, **kw):
    proc = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert proc.returncode == 0, f"{' '.join(cmd)}\n{proc.stdout[-4000:]}\n{proc.stderr[-4000:]}"
    return proc


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    if len(objs) < len(glob.glob(os.path.join(PKG, "csrc", "*.hip"))):
        from test_activation_aware_amd.build import build
        build()
        objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    out = tmp_path_factory.mktemp("asan")
    api_o = str(out / "api.o")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o])
    lib = str(out / "libttq_asan.so")
    _run(["g++", "-shared", *SAN, "-o", lib, api_o, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    return out, lib


def test_driver_under_sanitizers(asan_lib):
    out, lib = asan_lib
    exe = str(out / "driver")
    _run(["g++", "-std=c++17", "-g", *SAN, "-pthread", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "host_asan_driver.cpp"), lib, "-Wl,-rpath," + str(out), "-o", exe])
    proc = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert proc.stdout.strip().endswith("ALL OK"), proc.stdout[-2000:]


def test_host_abi_tests_under_sanitizers(asan_lib):
    _, lib = asan_lib
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(libasan), "libasan.so not found"
    # the interpreter is not instrumented: the runtime is preloaded, and leak
    # detection (which would report the interpreter's own allocations) is off
    proc = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                 os.path.join(ROOT, "tests", "test_abi_host.py")],
                cwd=ROOT, env=_env(LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                                   TTQ_LIBRARY=lib))
    assert " passed" in proc.stdout, proc.stdout[-2000:]
