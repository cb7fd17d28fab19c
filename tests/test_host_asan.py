"""The host code under AddressSanitizer, on the CPU.

Two ASan builds go to a temporary directory: the C ABI's host code (api.hip and segments.hip: all
argument checks, the workspace planning and the no-allocation scratch bookkeeping; the kernel
launchers replaced by tests/asan/launch_stubs.hip) and the fp64 oracle (oracle/gdn_oracle.c, with
its threads and heap buffers).  tests/test_abi_cpu.py and tests/test_oracle_pins.py then run in a
child process with the ASan runtime preloaded and the two builds in place of the usual libraries;
any ASan report fails the test.  The device code is not instrumented (no device sanitizer here).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_sequence_rule_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    for pat in ("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm-*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])


@pytest.fixture(scope="module")
def asan_builds(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("clang ASan runtime or ROCm compilers not found")
    d = tmp_path_factory.mktemp("asan")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "segments.hip"),
                os.path.join(ROOT, "tests", "asan", "launch_stubs.hip")):
        obj = str(d / (os.path.basename(src) + ".o"))
        _run([HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", *san, "-c", src, "-o", obj])
        objs.append(obj)
    lib = str(d / "libgdn.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o", lib, *objs])
    orc = str(d / "libgdn_oracle.so")
    _run([CLANG, "-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared", "-fsanitize=address",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", orc, "-lpthread", "-lm"])
    return rt, lib, orc


def test_abi_and_oracle_under_asan(asan_builds):
    rt, lib, orc = asan_builds
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:detect_odr_violation=0",
               GDN_TEST_LIBGDN=lib, GDN_TEST_ORACLE=orc, HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout
