"""Host code of the C ABI (lra_api.cpp: validation, planning and dispatch) built by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU, with stub kernel
launchers (tests/native/plan_check.cpp): the planner's checks plus every validation path."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GXX = "g++"
ROCM_INC, ROCM_LIB = "/opt/rocm/include", "/opt/rocm/lib"


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM_INC, "hip", "hip_runtime.h")),
                    reason="HIP headers not available")
def test_planner_and_validation_under_address_and_undefined_sanitizers(tmp_path):
    """Any sanitizer report, a failed check or a non-zero exit fails the test."""
    csrc = os.path.join(ROOT, "shared_rank_kv_amd", "csrc")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
             "-I", csrc]
    objs = []
    for src in (os.path.join(csrc, "lra_api.cpp"), os.path.join(ROOT, "tests", "native",
                                                                  "plan_check.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([GXX, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "plan_check_san")
    r = subprocess.run([GXX, "-fsanitize=address,undefined", *objs, "-o", exe, "-L", ROCM_LIB,
                        "-lamdhip64", f"-Wl,-rpath,{ROCM_LIB}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "planner checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
