"""Build libfsdp_shard.so in-tree with hipcc for gfx950.

Flags that matter for the arithmetic:
  -ffp-contract=off          no FMA contraction (each fp32 op rounds once)
  (default) correctly rounded fp32 divide and sqrt; fp32 subnormals preserved
  -target-feature -packed-fp32-ops   no packed fp32 instructions
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfsdp_shard.so")
SOURCES = [os.path.join(CSRC, "fsdp_kernels.hip"), os.path.join(CSRC, "fsdp_abi.cpp"),
           os.path.join(CSRC, "fsdp_ckpt.cpp"), os.path.join(CSRC, "fsdp_offload.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(extra_flags=(), out=LIB, verbose=False):
    """Compile every HIP source of the package into one shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra_flags) + ["-x", "hip"] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
