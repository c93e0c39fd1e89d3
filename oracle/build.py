"""Build the fp64 CPU oracle (``liboracle.so``) with gcc.

Test infrastructure: the library this builds is loaded only by the tests, the
smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it and return its path.

    Plain -O2: no -ffast-math, so every fp64 operation keeps IEEE semantics
    and the order written in the source.
    """
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
