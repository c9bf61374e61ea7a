"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Host code only (gcc): `oracle_sanitized_check.c` includes the oracle's C
source and runs quantization, silu, the GEMM at the INT32 closed forms
(K = 65536 and the largest accepted K with -128 * -128), the dequant and the
bf16 rounding; any out-of-bounds access or undefined behaviour aborts.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_is_clean_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitized_check"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "oracle_sanitized_check.c"), "-o", str(exe), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("host compiler lacks the sanitizer runtimes: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "sanitized oracle run: ok" in res.stdout
