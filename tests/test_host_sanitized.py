"""The C-ABI layer built for the host alone under the address and undefined-
behaviour sanitizers, with the stand-in device layer of
tests/host_check/stub_device.cpp in place of the kernels, and the ABI tests
(tests/test_abi.py: every validation and error path, the workspace planning,
the host Lloyd-Max tables) run against that build in a child process.  A heap
or stack overflow, a use after free, a signed overflow, a misaligned access or
a bad shift anywhere on those paths aborts the child and fails this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_cache_decode_pgkq_amd", "csrc")


def _gxx():
    return shutil.which("g++")


def _runtime(name):
    r = subprocess.run([_gxx(), f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not _gxx() or not _runtime("libasan.so"):
        pytest.skip("g++ with the address sanitizer runtime is not available")
    out = str(tmp_path_factory.mktemp("hostcheck") / "libpgkq_hostcheck.so")
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(ROOT, "tests", "host_check", "stub_device.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_sanitized_build_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", sanitized_lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    assert "pgkq_decode_attn" in syms and "pgkq_hostcheck_calls" in syms


def test_abi_error_paths_under_sanitizers(sanitized_lib):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    # the sanitizer runtime has to come first among the preloaded libraries
    env["LD_PRELOAD"] = _runtime("libasan.so") + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PGKQ_LIB"] = sanitized_lib
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout and "skipped" not in r.stdout, tail
