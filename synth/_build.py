"""Builds the two generator libraries in place (gcc for the host, hipcc for gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    host = os.path.join(HERE, "libsynth_host.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", host,
                    os.path.join(HERE, "synth_host.c")], check=True)
    dev = os.path.join(HERE, "libsynth_dev.so")
    subprocess.run(["hipcc", *HIP_FLAGS, "-o", dev, os.path.join(HERE, "synth_dev.hip")],
                   check=True, stderr=None if verbose else subprocess.DEVNULL)
    return [host, dev]


if __name__ == "__main__":
    print(build(verbose=True))
