"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the host-sanitizer build, then the
C-ABI host tests (validation of every entry point, workspace queries,
zoned planning against the oracle's layout, corrupted and truncated plans)
in a child process with the sanitizer runtime preloaded.  Any report ends
the child with a non-zero status."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_abi_host_tests_under_host_sanitizers():
    if not (os.path.exists(CLANG) and os.path.exists(HIPCC)):
        pytest.skip("ROCm clang / hipcc not installed")
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(rt) and os.path.exists(rt)):
        pytest.skip("AddressSanitizer runtime not found")
    script = os.path.join(ROOT, "dequant_decode_attention_amd", "build_host_sanitize.py")
    r = subprocess.run([sys.executable, script], cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    lib = os.path.join(ROOT, "dequant_decode_attention_amd", "libdqattn_san.so")
    env = dict(os.environ, LD_PRELOAD=rt, DQA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child loads the instrumented build
    probe = subprocess.run([sys.executable, "-c",
                            "import dequant_decode_attention_amd as d; print(d.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_host.py", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
