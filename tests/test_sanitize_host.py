"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds libhla_san.so (sanitizers on the host code only) and runs the host-side
ABI tests against it in a child process with the shared sanitizer runtime
preloaded: every validation path, the workspace queries and the RoPE table
helper, with no kernel launched. Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_code_is_clean_under_asan_and_ubsan():
    from softmax_attention_relu_amd import build_sanitize

    lib = build_sanitize.build()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": build_sanitize.runtime(), "HLA_LIBRARY": lib,
                "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_host.py", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in r.stdout, out[-4000:]
