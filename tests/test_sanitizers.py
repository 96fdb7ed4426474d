"""CPU sanitizer builds (no GPU): the oracle and the library's host-side code
compiled with AddressSanitizer and UndefinedBehaviorSanitizer and run clean.

  * the oracle (oracle/mustafar_oracle.cpp) is built as a sanitized shared
    library and every CPU pin of it (test_oracle_pins.py, test_oracle_append.py)
    runs against that build in a child process with the sanitizer runtimes
    preloaded; any report aborts the child;
  * the C ABI (api.hip: argument checks, byte accounting, split and workspace
    sizing) is built for the host only with the same sanitizers, kernel
    launchers stubbed, and driven through every error path by
    tests/sanitize/abi_host_driver.cpp.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-pthread",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "mustafar_oracle.cpp"), "-o", str(lib)], check=True)
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=f"{asan}:{ubsan}", MUSTAFAR_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_append.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="no hipcc")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_host"
    csrc = os.path.join(ROOT, "unstructured_sparse_kv_amd", "csrc")
    san = os.path.join(ROOT, "tests", "sanitize")
    # sanitizers on the host side only (-Xarch_host before each); api.hip's device
    # part is only the no-alloc scratch array
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-Wno-unused-command-line-argument",
                    os.path.join(csrc, "api.hip"), os.path.join(san, "launch_stubs.cpp"),
                    os.path.join(san, "abi_host_driver.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], env=dict(os.environ, **SAN_ENV), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "all passed" in r.stdout
