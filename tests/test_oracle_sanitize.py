"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) runs every entry point without a report: no
out-of-bounds access, leak or undefined behaviour in the checker itself."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "attn_oracle.c"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", exe, "-lm"]
    subprocess.check_call(cmd)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout, res.stderr)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stderr[-3000:]
