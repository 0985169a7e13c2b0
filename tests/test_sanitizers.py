"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle, compiled with gcc together with a C driver that hands it heap
  buffers of exactly the sizes its layout needs (tests/c/oracle_sanitized.c),
  so any byte touched outside them, any leak and any undefined operation fails
  the run.
* The host side of libkvpub (argument checks, all-or-nothing paths that need
  no device), built with the sanitizers on its host pass only and driven by the
  plain C99 program of the ABI test (tests/c/abi_from_c.c).  The kernels are
  built as usual: GPU code is never built with a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS_C = os.path.join(ROOT, "tests", "c")

# Same IEEE binary32 semantics as the oracle's own build.
ORACLE_FP_FLAGS = ["-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard"]


def _run(cmd, env=None, timeout=300):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    build = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", *ORACLE_FP_FLAGS,
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             os.path.join(TESTS_C, "oracle_sanitized.c"), os.path.join(ROOT, "oracle", "kvpub_oracle.c"),
             "-o", exe]
    r = _run(build)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(_hipcc()), reason="hipcc not available")
def test_host_library_under_asan_and_ubsan(tmp_path):
    from replicated_fp8_sparse_amd import build as B

    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = str(tmp_path / "libkvpub_san.so")
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        r = _run([_hipcc(), *B.HIPFLAGS, *host_san, "-c", os.path.join(B.CSRC, src), "-o", obj], timeout=600)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    r = _run([_hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", lib])
    assert r.returncode == 0, r.stderr
    os.symlink(lib, str(tmp_path / "libkvpub.so"))
    exe = str(tmp_path / "abi_from_c_san")
    r = _run([clang, "-std=c99", "-Wall", "-Werror", "-g", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", os.path.join(TESTS_C, "abi_from_c.c"), "-I",
              os.path.join(ROOT, "include"), "-L", str(tmp_path), "-lkvpub", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    assert r.returncode == 0, r.stderr
    # The HIP runtime's own start-up allocations are not this library's: leak
    # checking is off for this run; out-of-bounds and undefined behaviour abort.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
