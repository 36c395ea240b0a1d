"""The library's host code (argument validation, size arithmetic, launch set-up)
built with AddressSanitizer and UndefinedBehaviorSanitizer, then driven through
every validation path of tests/test_abi.py.  Only the host side is instrumented:
each -fsanitize flag is passed to hipcc after -Xarch_host, so the device code is
built as usual.  No GPU is needed; every call fails validation before any HIP
launch."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(_asan_runtime() is None, reason="needs the ROCm clang AddressSanitizer runtime")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    from fp4_quantization_precision_amd import build as b
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([b.HIPCC, *b.COMMON, *san, "-x", "hip", "-c", os.path.join(b.CSRC, src),
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(b.SOURCES))) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = str(tmp_path / "libtq_sanitized.so")
    r = subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC",
                        "-fsanitize=address,undefined", "-shared-libasan", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    runner = (
        "import sys; sys.path.insert(0, %r)\n"
        "import fp4_quantization_precision_amd._lib as l; l.LIB_PATH = %r\n"
        "import pytest\n"
        "raise SystemExit(pytest.main(['-q', '-p', 'no:cacheprovider', %r, "
        "'-k', 'not exports and not host_tensors']))\n" % (ROOT, lib, os.path.join(HERE, "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", runner], capture_output=True, text=True, env=env,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert " passed" in r.stdout
