"""The oracle (oracle.c) and the input generator (synth.c) built for the CPU
with AddressSanitizer and UndefinedBehaviorSanitizer, driven over small,
ragged and empty-share inputs by tests/sanitize/driver.c: no out-of-bounds
access, leak or undefined behaviour (CPU only)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(HERE, "sanitize", "driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
