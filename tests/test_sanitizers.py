"""Host-code sanitizer builds (no GPU): the CPU oracle and the C ABI's host
paths, built with AddressSanitizer + UndefinedBehaviorSanitizer and run on
drivers that reach every entry point (tests/oracle_sanitize_check.c,
tests/abi_sanitize_check.cpp).  Any out-of-bounds access, leak or undefined
operation makes the driver exit non-zero with the sanitizer's report.  On the
HIP sources only the host compilation is instrumented (each -fsanitize= goes
after -Xarch_host); the device code is built as usual."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from conditional_draft_tree_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan",
          "-o", exe, os.path.join(TESTS, "oracle_sanitize_check.c"), os.path.join(ROOT, "oracle", "dtree_oracle.c"),
          "-lm"])
    r = _run([exe], env=SAN_ENV)
    assert "ran clean" in r.stdout


CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(libbuild.HIPCC) and os.path.exists(CLANGXX)), reason="needs the ROCm compilers")
def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", f]
    flags = [f for f in libbuild.FLAGS if f != "-O3"] + ["-O1", "-g"] + host_san
    srcs = sorted(f for f in os.listdir(libbuild.CSRC) if f.endswith(".hip"))

    def compile_one(name):
        obj = str(tmp_path / (name + ".o"))
        _run([libbuild.HIPCC, *flags, *libbuild.FILE_FLAGS.get(name, []), "-c", os.path.join(libbuild.CSRC, name),
              "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_check.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", "-c",
          os.path.join(TESTS, "abi_sanitize_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    _run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=SAN_ENV)
    assert "ran clean" in r.stdout
