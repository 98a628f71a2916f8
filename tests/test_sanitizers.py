"""The host structure builder and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Each test builds a small driver (tests/sanitize/) together with the source
it checks, with g++ or gcc and -fsanitize=address,undefined (no recovery:
the first finding aborts), and runs it. The structure driver builds
structures for many valid and malformed masks and walks every host entry
point; the oracle driver runs every oracle entry point on small inputs,
including empty rows, empty columns and a structure with no stored block.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, tmp_path, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr
    return run.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_structure_builder_clean_under_asan_ubsan(tmp_path):
    exe = tmp_path / "structure_driver"
    cmd = ["g++", "-std=c++17", *SAN, "-I", str(ROOT / "include"),
           "-I", str(ROOT / "block_sparse_attention_bsr_amd" / "csrc"),
           str(ROOT / "tests" / "sanitize" / "structure_driver.cpp"),
           str(ROOT / "block_sparse_attention_bsr_amd" / "csrc" / "structure.cpp"), "-o", str(exe)]
    out = _run(cmd, tmp_path, exe)
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", "-fopenmp", *SAN, str(ROOT / "tests" / "sanitize" / "oracle_driver.c"),
           str(ROOT / "oracle" / "bsr_attn_oracle.c"), "-o", str(exe), "-lm"]
    out = _run(cmd, tmp_path, exe)
    assert "ok" in out
