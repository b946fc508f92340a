"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only), driven through every entry point on small inputs by
tests/oracle_sanitize_main.c: no out-of-bounds access, leak or undefined
behaviour in the reference the GPU path is checked against."""
import os
import shutil
import subprocess

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math",
           "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           obuild.SRC, os.path.join(HERE, "oracle_sanitize_main.c"), "-o", str(exe), "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "every call ok" in run.stdout
