"""The host tests (tests/test_abi_host.py: the packer's bit layouts over
caller buffers, the layout arithmetic, every refusal path of the C ABI) run
again against a build of the host sources with AddressSanitizer and
UndefinedBehaviorSanitizer (build_host_sanitized: g++ only, the device entry
points replaced by refusals), in a child process with the sanitizer
runtimes preloaded; any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_tests_pass_under_asan_and_ubsan():
    from quantized_routed_expert_fp32_amd.csrc import build as B
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("the sanitizer runtimes are not installed with g++")
    lib = B.build_host_sanitized()
    env = dict(os.environ)
    env.update(MOE_LIBRARY=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
