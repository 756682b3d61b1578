"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

api.cpp, nf4_table.cpp and plan.cpp are built with g++ -fsanitize=address,undefined into a
library whose kernel launchers are stubs (tests/host/launch_stubs.cpp): every host check
of the ABI runs before a launch.  The launch planners' unit-check program (tests/host/plan_units.cpp)
runs under the same sanitizers, and the ABI host tests (tests/test_abi_host.py) run against
that library in a child process with the ASan runtime preloaded.  Any sanitizer report fails
the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_lora_fine_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
GXX = shutil.which("g++")

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
COMMON = ["-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}

pytestmark = pytest.mark.skipif(GXX is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                                reason="needs g++ and the HIP host runtime")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-6000:]}"
    return r.stdout


@pytest.fixture(scope="module")
def san_build(tmp_path_factory):
    out = tmp_path_factory.mktemp("san")
    srcs = [os.path.join(CSRC, f) for f in ("api.cpp", "nf4_table.cpp", "plan.cpp")] + \
           [os.path.join(HOST, "launch_stubs.cpp")]
    lib = str(out / "libnf4lora_san.so")
    _run([GXX, *COMMON, *SAN, "-shared", "-o", lib, *srcs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    units = str(out / "plan_units")
    _run([GXX, *COMMON, *SAN, "-o", units, os.path.join(HOST, "plan_units.cpp"), os.path.join(CSRC, "plan.cpp")])
    return lib, units


def test_plan_units_sanitized(san_build):
    _, units = san_build
    out = _run([units], env={**os.environ, **SAN_ENV})
    assert "plan units: ok" in out


def test_abi_host_checks_sanitized(san_build):
    lib, _ = san_build
    asan = subprocess.run([GXX, "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    env = {**os.environ, **SAN_ENV, "NF4LORA_LIB": lib, "LD_PRELOAD": asan}
    out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                os.path.join(ROOT, "tests", "test_abi_host.py")], env=env, cwd=ROOT)
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
