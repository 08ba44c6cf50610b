"""Builds the sanitized host-only fuzz program of the C ABI: capi.cpp and
plan.cpp with the launcher stand-ins of stub_launch.cpp, compiled by g++
with AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no HIP
source and no GPU code is part of this build)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "yarn_rope_kv_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "capi_host")
EXE = os.path.join(OUT_DIR, "capi_fuzz")
SOURCES = [os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "fuzz_main.cpp")]


def build():
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++20", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", *SOURCES, "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed:\n{' '.join(cmd)}\n{r.stderr}")
    return EXE


if __name__ == "__main__":
    print(build())
