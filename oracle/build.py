"""Builds liboracle.so from oracle.c with the host C compiler.

Test infrastructure: the oracle is compiled plain (-O2, IEEE arithmetic, no
fast-math, no explicit SIMD) and threaded with OpenMP over whole outputs only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(out=LIB, extra_flags=()):
    """Compile oracle.c into `out`; `extra_flags` lets a test add -D options."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-fopenmp", *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
