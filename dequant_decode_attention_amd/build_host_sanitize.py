"""Host-sanitizer build of libdqattn, for CPU runs only.

The host code (argument validation, workspace queries, zoned planning and
plan checking, launch set-up) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer; the gfx950 device code is compiled exactly as
in build.py and is not instrumented.  The result is
dequant_decode_attention_amd/libdqattn_san.so (objects under _build_san/).

Usage: python dequant_decode_attention_amd/build_host_sanitize.py

Run the C-ABI host tests against it (the interpreter is not instrumented,
so the sanitizer runtime is preloaded; DQA_LIBRARY makes the binding load
this build):

  LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \\
  ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 \\
  UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
  DQA_LIBRARY=$PWD/dequant_decode_attention_amd/libdqattn_san.so \\
  python -m pytest tests/test_abi_host.py -m "not gpu"

tests/test_host_sanitizer.py does both steps.
"""
import concurrent.futures as cf
import glob
import importlib.util
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build_san")
LIB = os.path.join(HERE, "libdqattn_san.so")

_spec = importlib.util.spec_from_file_location("_dqattn_build", os.path.join(HERE, "build.py"))
_b = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_b)

# every sanitizer option applies to the host compilation only
HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    r = subprocess.run([_b.HIPCC] + _b.DEVICE_FLAGS + HOST_FLAGS + ["-c", src, "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj


def build(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(_b.CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, srcs))
    # the sanitizer runtime is not linked in: it is preloaded into the process
    tmp = LIB + ".tmp"
    r = subprocess.run([_b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
