"""Compile the oracle's plain C into a shared library (gcc, -O2, OpenMP,
no fast-math).  Test infrastructure only."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(_HERE, "bqref.c")
    out = os.path.join(_HERE, "liboracle_bqref.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-Wall", "-Werror", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
