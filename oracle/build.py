"""Builds the fp64 CPU oracle (test infrastructure) into oracle/libkda_oracle.so with gcc.

Only tests, the smoke check and the CPU-baseline leg of the benchmark use the
oracle; the product library never links or loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


SAN_LIB = os.path.join(HERE, "libkda_oracle_san.so")
FLAGS = ["-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror", "-fno-fast-math",
         "-ffp-contract=off"]
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (host code only: the
# oracle is plain C), loaded by the sanitizer test through KDA_ORACLE_LIB with libasan preloaded
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _compile(out, opt):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc"] + opt + FLAGS + [SRC, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile kda_oracle.c; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    return _compile(LIB, ["-O2"])


def build_sanitized() -> str:
    """Compile kda_oracle.c with AddressSanitizer and UBSan; returns the library path."""
    return _compile(SAN_LIB, SAN_FLAGS)


if __name__ == "__main__":
    print(build())
