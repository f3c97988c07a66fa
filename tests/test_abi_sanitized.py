"""The C ABI's argument checking under host AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): api.cpp is built with the
sanitizers on its host code against launcher stubs, and a driver walks the
refusal paths of every entry point (fake device pointers, never
dereferenced; real host segment and problem tables).  Also checks that
every error-message format in api.cpp uses only the conversions passed to
it (a bare '%' in a format is undefined behaviour)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_error_formats_use_only_passed_conversions():
    src = open(os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "csrc", "api.cpp")).read()
    formats = re.findall(r'fail\(\s*FP4Q_[A-Z_]+\s*,\s*"((?:[^"\\]|\\.)*)"', src)
    assert len(formats) > 40
    for fmt in formats:
        for m in re.finditer(r"%", fmt):
            rest = fmt[m.start():]
            assert re.match(r"%(s|d|lld|%)", rest) or fmt[m.start() - 1] == "%", fmt


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("ld") is None, reason="no hipcc")
def test_abi_refusals_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_sanitized")
    srcs = [os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "csrc", "api.cpp"),
            os.path.join(ROOT, "tests", "abi_sanitize", "stubs.cpp"),
            os.path.join(ROOT, "tests", "abi_sanitize", "driver.cpp")]
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-g", "-O1",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I" + os.path.join(ROOT, "include"), *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert r.stdout.startswith("ok "), out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
