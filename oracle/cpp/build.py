"""Build the C++ oracle (test infrastructure only): oracle/cpp/libnvfp4_oracle.so.

    python oracle/cpp/build.py

g++ with OpenMP, for any x86-64-v3 host (AVX2 + FMA), so the library built
here also runs on the GPU machine's host.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.cpp")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")
FLAGS = ["-O3", "-std=gnu++17", "-march=x86-64-v3", "-mtune=generic", "-fopenmp", "-fPIC",
         "-shared", "-Wall"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    r = subprocess.run(["g++", *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stdout + r.stderr)
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
