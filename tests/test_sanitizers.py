"""Sanitizer builds on the CPU (no GPU): the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, and every source of libfsdp_shard.so -- host part
instrumented, device code as usual -- under ASan + UBSan and under
ThreadSanitizer, each driven by a program in tests/sanitize/:
  * oracle_checks.c: every oracle function on buffers of exact size;
  * host_checks.cpp "all": argument validation of every entry point, launch
    planning with never-dereferenced device pointers (2^26-element slices,
    packed tables, N = 128, 16-bit state, every optimizer, segmented
    flatten/unflatten), CRC32C against a bitwise reference at every offset,
    the threaded host AdamW, and the shard-file reader fed every truncation
    and a bit flip at every header and table byte;
  * host_checks.cpp "threads" (TSan): the host AdamW worker pool at 3 and 16
    threads and CRC32C from 8 threads at once.
Any sanitizer report fails the run.  The builds go to a temporary directory.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sharded_state_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_SOURCES = ["fsdp_kernels.hip", "fsdp_units_adamw.hip", "fsdp_units_sgd.hip", "fsdp_units_adamax.hip",
               "fsdp_units_adadelta.hip", "fsdp_abi.cpp", "fsdp_ckpt.cpp", "fsdp_offload.cpp"]
COMMON = ("-O1 -g -fno-omit-frame-pointer -std=c++17 --offload-arch=gfx950 -ffp-contract=off "
          "-Xclang -target-feature -Xclang -packed-fp32-ops").split() + ["-I", os.path.join(ROOT, "include"),
                                                                       "-I", CSRC]
# sanitizers on the host part only: each flag right after -Xarch_host
HOST_ASAN_UBSAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined " \
                  "-Xarch_host -fno-sanitize-recover=all".split()
HOST_TSAN = "-Xarch_host -fsanitize=thread".split()

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(HIPCC),
                                reason="needs gcc and hipcc")


def _run(cmd, env=None, timeout=900):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\nexit %d\n%s\n%s" % (" ".join(cmd), r.returncode, r.stdout[-4000:], r.stderr[-8000:])
    return r


def _build_host(out_dir, san, tag):
    """Every library source and the host driver, compiled in parallel and linked."""
    srcs = [os.path.join(CSRC, f) for f in LIB_SOURCES] + [os.path.join(HERE, "host_checks.cpp")]
    objs = [os.path.join(out_dir, "%s_%s.o" % (tag, os.path.basename(s))) for s in srcs]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 4), 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC] + COMMON + san + ["-x", "hip", "-c", so[0], "-o", so[1]]),
                    zip(srcs, objs)))
    exe = os.path.join(out_dir, "host_checks_" + tag)
    _run([HIPCC, "--offload-arch=gfx950"] + san + objs + ["-o", exe])
    return exe


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "fsdp_oracle.c"), os.path.join(HERE, "oracle_checks.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([exe], env=env)
    assert "oracle sanitizer checks: ok" in r.stdout


def test_host_layer_under_asan_and_ubsan(tmp_path):
    exe = _build_host(str(tmp_path), HOST_ASAN_UBSAN, "asan")
    work = tmp_path / "files"
    work.mkdir()
    # the HIP runtime keeps allocations until exit: leak reports would be its own
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = _run([exe, "all", str(work)], env=env)
    assert "host sanitizer checks (all)" in r.stdout
    assert "launch planning with fake pointers skipped" not in r.stdout


def test_host_layer_under_tsan(tmp_path):
    exe = _build_host(str(tmp_path), HOST_TSAN, "tsan")
    work = tmp_path / "files"
    work.mkdir()
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1", HIP_VISIBLE_DEVICES="")
    r = _run([exe, "threads", str(work)], env=env)
    assert "host sanitizer checks (threads)" in r.stdout
