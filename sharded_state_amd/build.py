"""Build libfsdp_shard.so in-tree with hipcc for gfx950.

Flags that matter for the arithmetic:
  -ffp-contract=off          no FMA contraction (each fp32 op rounds once)
  (default) correctly rounded fp32 divide and sqrt; fp32 subnormals preserved
  -target-feature -packed-fp32-ops   no packed fp32 instructions
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfsdp_shard.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "fsdp_kernels.hip", "fsdp_units_adamw.hip", "fsdp_units_sgd.hip", "fsdp_units_adamax.hip",
    "fsdp_units_adadelta.hip", "fsdp_abi.cpp", "fsdp_ckpt.cpp", "fsdp_offload.cpp")]
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(extra_flags=(), out=LIB, verbose=False, jobs=None):
    """Compile every source of the package (in parallel, one object each) and
    link them into one shared library."""
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.basename(src) + "." + tag + ".o")
        objs.append(obj)
        cmds.append([HIPCC] + FLAGS + list(extra_flags) + ["-x", "hip", "-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 4), 16)
    try:
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for cmd in cmds:
                if verbose:
                    print(" ".join(cmd), file=sys.stderr)
            list(ex.map(lambda c: subprocess.run(c, check=True), cmds))
        tmp = out + ".tmp" + tag
        link = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(link), file=sys.stderr)
        subprocess.run(link, check=True)
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
