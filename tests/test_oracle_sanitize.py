"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code, gcc), driven through
every entry point on small inputs, edge cases included (tests/oracle_sanitize_driver.c). CPU only."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the oracle")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_san")
        subprocess.run(["gcc", "-O1", "-g", "-std=gnu11", "-ffp-contract=off", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", ORACLE,
                        os.path.join(ORACLE, "nvfp4_oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
                        "-o", exe, "-lm"], check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle sanitizer run: ok" in r.stdout
        assert "runtime error" not in r.stderr, r.stderr
