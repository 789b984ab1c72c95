"""The C ABI's host code (argument checks, workspace planning, dispatch) built
with AddressSanitizer and UndefinedBehaviorSanitizer, driven by
``tests/host/validator_check.cpp`` over extreme and defective arguments
(CPU only: every call there is a size query or is refused before any HIP
call).  The device objects are linked unchanged; only the host translation
unit and the driver are instrumented.  Leak checking is off: the HIP runtime
keeps allocations until exit."""

import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dequant_gemv_rht_amd", "_lib")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
INC = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_validator_under_asan_ubsan(tmp_path):
    objs = sorted(o for o in glob.glob(os.path.join(LIB, "*.o")) if not o.endswith("api.cpp.o"))
    if not objs:
        pytest.fail("the library's objects are not built: run python -m dequant_gemv_rht_amd.build")
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "validator_check.o")
    exe = str(tmp_path / "validator_check")
    _run(["g++", "-std=c++17", "-g", "-O1", *SAN, *INC, "-c",
          os.path.join(ROOT, "dequant_gemv_rht_amd", "csrc", "api.cpp"), "-o", api])
    _run(["g++", "-std=c++17", "-g", "-O1", *SAN, *INC, "-c",
          os.path.join(ROOT, "tests", "host", "validator_check.cpp"), "-o", drv])
    _run(["g++", *SAN, drv, api, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=600)
    assert "checked" in r.stdout
