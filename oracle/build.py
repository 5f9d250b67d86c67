"""Build the oracle's shared library with gcc (test infrastructure only)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build_oracle():
    """Compile oracle.c -> liboracle.so: -O2, OpenMP, IEEE semantics (no
    fast-math, no contraction into fused multiply-adds)."""
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_oracle())
