"""Build the CPU oracle shared library (test infrastructure only).

The oracle is plain C compiled with gcc: -O2, no FMA contraction, no fast-math,
so every float operation in it is one IEEE-754 binary32 operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fsdp_oracle.c")
LIB = os.path.join(HERE, "libfsdp_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-Wall", "-Wextra"]


def build(force=True):
    """Compile oracle/fsdp_oracle.c into oracle/libfsdp_oracle.so."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc"] + CFLAGS + ["-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
