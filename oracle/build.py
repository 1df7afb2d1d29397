"""Build the CPU oracle (oracle/q8ref.c) into oracle/libq8ref.so with gcc.

Test infrastructure only: see oracle/__init__.py.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q8ref.c")
LIB = os.path.join(HERE, "libq8ref.so")

# -ffp-contract=off: the quantiser's multiply must not fuse with anything.
# No -ffast-math, no intrinsics: binary32 divides stay correctly rounded.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
