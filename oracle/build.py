"""Builds the fp64 CPU oracle (test infrastructure) into oracle/libkda_oracle.so with gcc.

Only tests, the smoke check and the CPU-baseline leg of the benchmark use the
oracle; the product library never links or loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(force: bool = True) -> str:
    """Compile kda_oracle.c; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
