"""The library's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Every library source and tests/host/sanitize_driver.cpp are compiled with
the sanitizers on the host pass only (hipcc -Xarch_host -fsanitize=...; the
device code is built as usual) and linked into one executable, which feeds
the C ABI NULL pointers, out-of-range configurations and bad sizes and
checks that each call returns its documented status and message before any
device call, with no sanitizer report."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "swiftkv_prefill_skipping_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_validation_under_asan_and_ubsan():
    from swiftkv_prefill_skipping_amd import build as b
    tmp = tempfile.mkdtemp(prefix="skv_san_")
    try:
        flags = [f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                 "-Xclang", "-packed-fp32-ops", *SAN]

        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        srcs = [os.path.join(CSRC, s) for s in b.SOURCES] + [os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp")]
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, srcs))
        exe = os.path.join(tmp, "sanitize_driver")
        r = subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", *SAN, *objs, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = r.stdout + r.stderr
        assert r.returncode == 0 and "ALL OK" in r.stdout, out[-4000:]
        assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
