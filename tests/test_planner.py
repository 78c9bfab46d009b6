"""The attention planner (host code of the C ABI), exercised on the CPU: tests/native/
plan_check.cpp is compiled with lra_api.cpp and stub kernel launchers, and run."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_planner_units_and_launches(tmp_path):
    csrc = os.path.join(ROOT, "shared_rank_kv_amd", "csrc")
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
             "-I", os.path.join(ROOT, "include"), "-I", csrc]
    objs = []
    for src in (os.path.join(csrc, "lra_api.cpp"), os.path.join(ROOT, "tests", "native",
                                                                  "plan_check.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "plan_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "planner checks passed" in r.stdout

