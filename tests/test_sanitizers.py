"""Host sanitizers. The CPU oracle and the library's host-side table checks
are built a second time with gcc/g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (every report fatal), and their CPU tests run
against those builds in a fresh process (the ASan runtime preloaded, since
the Python interpreter is not instrumented). Any out-of-bounds access, use
after free, signed overflow, bad shift or out-of-range float conversion in
that code fails the test. Device code is not built this way: the GPU
kernels are checked by the parity tests and by the host-side checks of
their arguments."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
       "-fno-sanitize-recover=all", "-fPIC", "-shared", "-pthread"]
ORACLE_PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_readings.py", "tests/test_oracle_ops.py",
               "tests/test_oracle_contiguous.py", "tests/test_oracle_attention.py", "tests/test_oracle_fast_math.py"]


def asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not path or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def run_under_sanitizers(env_var, lib, tests, tmp_path):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", env_var: lib})
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-n", "4"] + tests
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math"] + SAN +
                   [os.path.join(ROOT, "oracle", "kvfp4_oracle.c"), "-o", lib, "-lm"], check=True)
    run_under_sanitizers("KVFP4_ORACLE_LIB", lib, ORACLE_PINS, tmp_path)


def test_table_checks_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libtable_checks_sanitized.so")
    subprocess.run(["g++", "-std=c++17"] + SAN +
                   [os.path.join(ROOT, "kv_cache_quantization_paged_amd", "csrc", "table_checks.cpp"), "-o", lib],
                   check=True)
    run_under_sanitizers("KVFP4_TABLE_CHECKS_LIB", lib, ["tests/test_table_checks.py", "-k", "raw"], tmp_path)


def test_a_planted_overflow_is_caught(tmp_path):
    """the harness itself: an out-of-bounds read planted in a copy of the
    table checks must fail under the sanitizers"""
    src = open(os.path.join(ROOT, "kv_cache_quantization_paged_amd", "csrc", "table_checks.cpp")).read()
    planted = src.replace("for (int32_t b = 0; b < batch; ++b)\n        if (indptr[b + 1] < indptr[b])",
                          "for (int32_t b = 0; b <= batch; ++b)\n        if (indptr[b + 1] < indptr[b])")
    assert planted != src
    path = tmp_path / "table_checks_planted.cpp"
    path.write_text(planted.replace('#include "../../include/kvfp4.h"', f'#include "{ROOT}/include/kvfp4.h"'))
    lib = str(tmp_path / "libplanted.so")
    subprocess.run(["g++", "-std=c++17"] + SAN + [str(path), "-o", lib], check=True)
    with pytest.raises(AssertionError):
        run_under_sanitizers("KVFP4_TABLE_CHECKS_LIB", lib, ["tests/test_table_checks.py", "-k", "raw"], tmp_path)
