"""The misaligned 16-bit piece loaders of the kernels (load8_u16_words and
load8_u16_tail in tiled_matrix_multiplication_amd/csrc/load_words.h,
compiled for the host from the same header) read nothing past the word (the
element) holding the last valid element, for every alignment and valid
count, and return the right values: tests/load_words_check.hip puts that
word (element) against a guard page."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_load8_u16_words_stays_before_the_guard_page(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "load_words_check")
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "tiled_matrix_multiplication_amd", "csrc"),
                    os.path.join(ROOT, "tests", "load_words_check.hip"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, f"rc {r.returncode}: {r.stdout} {r.stderr}"
    assert r.stdout.startswith("OK 29 windows"), r.stdout
