"""The library's host code and the C oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/host_check.cpp links smla_host.cpp against stubs of the kernel
launchers and of the few HIP runtime calls it makes, and drives every entry
point over a grid of shapes and plans, the argument errors, validate mode, the
workspace status word and the spin-limit knob; each stub touches the ends of
the buffers its kernel would, at the extents the arguments imply.
tests/sanitize/oracle_check.c runs every oracle entry point on edge-case
inputs.  Both are built here with gcc/g++ (host code only, no GPU code)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")
ENV.pop("SMLA_VALIDATE", None)
ENV.pop("SMLA_MERGE_SPIN_LIMIT", None)


def _run(exe):
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    text = r.stdout + r.stderr
    assert "runtime error" not in text and "AddressSanitizer" not in text and "LeakSanitizer" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    return text


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_check"
    subprocess.run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-o", str(exe), "-lm"], check=True)
    assert "0 failures" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include/hip"),
                    reason="g++ or the HIP headers not found")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(ROOT, "sparse_mla_top_amd", "csrc", "smla_host.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_check.cpp"), "-o", str(exe)], check=True)
    out = _run(exe)
    assert " 0 failures" in out
