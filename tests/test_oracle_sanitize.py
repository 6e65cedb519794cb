"""The oracle's C code built with AddressSanitizer and UndefinedBehavior-
Sanitizer (host code only, gcc) and run over every entry point, format and
operand layout on exactly-sized buffers (tests/oracle_sanitize_driver.c):
no access outside a buffer, no undefined behaviour, no leak, and the
results it knows exactly."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    flags = ["-O1", "-g", "-fopenmp", "-std=c99", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run([gcc, *flags, os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert r.stdout.strip().endswith("OK"), r.stdout
