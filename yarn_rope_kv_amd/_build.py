"""Builds libyrk.so in place: every HIP source for gfx950, then one link.

Device code is compiled with packed-fp32 instruction selection turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops).  The decode kernels keep
their MFMA accumulators in VGPRs (-amdgpu-mfma-vgpr-form): the NVFP4 split
kernel rescales its output accumulators with vector instructions every step,
which on AGPRs would cost a read and a write per element."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "yrk")
LIB = os.path.join(HERE, "libyrk.so")
SOURCES = ["capi.cpp", "plan.cpp", "rope.hip", "kv_append.hip", "decode.hip", "verify.hip",
           "prefill.hip", "noalloc.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "verify.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append(["hipcc", *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src),
                     "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB, *objs])
    return [LIB]


if __name__ == "__main__":
    print(build(verbose=True))
