"""The host half of the library (plan builder, plan cache, C ABI argument checks) built
with g++ under the address + undefined-behaviour sanitizers and, separately, the thread
sanitizer, and driven by ``tests/sanitize/host_driver.cpp``: a geometry sweep with every
introspection call at exact buffer sizes, cache eviction with handles outstanding, every
argument error path, and threads creating and releasing shared plans.  The kernel
launchers are host-only stubs (``tests/sanitize/stub_launch.cpp``); no device code is
built.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunk_windowed_softmax_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                                reason="needs g++ and the HIP runtime library")


def _build(tmp_path, name, flags):
    exe = tmp_path / name
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *flags,
           os.path.join(SAN, "host_driver.cpp"), os.path.join(SAN, "stub_launch.cpp"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-pthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    r = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    return r


def test_address_and_undefined_sanitizers(tmp_path):
    exe = _build(tmp_path, "host_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])
    _run(exe, env_extra={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})


def test_thread_sanitizer(tmp_path):
    exe = _build(tmp_path, "host_tsan", ["-fsanitize=thread"])
    r = _run(exe, "8", env_extra={"TSAN_OPTIONS": "halt_on_error=1"})
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr
