"""Build liblra.so in-tree with hipcc for gfx950.

    python -m shared_rank_kv_amd.build

compiles every source under csrc/ to objects in csrc/_build/ and links
shared_rank_kv_amd/liblra.so.  Always recompiles (the build is a few seconds per file).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "liblra.so")
SOURCES = ["lra_api.cpp", "fla_bf16.hip", "fla_decode.hip", "fla_f32.hip", "precompute.hip",
           "noalloc.hip", "expand.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          # packed fp32 VALU ops are kept out of the device code (see the design notes)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-result"]
# The attention kernels take no NaN inputs (masked scores are -inf, never NaN).  With the
# IEEE mode bit off, v_max_f32 needs no quieting of signalling NaNs, so the softmax row max
# does not canonicalise every MFMA result first.
EXTRA = {"fla_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
         "fla_decode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj, msgs


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (_, msgs), src in zip(results, SOURCES):
            for m in msgs:
                print(f"[{src}] {m}")
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
