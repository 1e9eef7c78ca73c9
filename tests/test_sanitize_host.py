"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the CPU oracle and the library's host repack (both plain C/C++, no HIP)
with gcc/g++ and -fsanitize=address,undefined, and runs a check program for
each (tests/sanitize/): any out-of-bounds access, leak or undefined behaviour
fails the run, as does any failed value check.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _sanitizers_available(tmp_path) -> bool:
    src = tmp_path / "probe.c"
    src.write_text("int main(void){return 0;}\n")
    r = subprocess.run(["gcc", *SAN, str(src), "-o", str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def _build_and_run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.fixture(scope="module")
def tmp(tmp_path_factory):
    p = tmp_path_factory.mktemp("san")
    if not shutil.which("gcc") or not _sanitizers_available(p):
        pytest.skip("gcc with the address and undefined-behaviour sanitizers is not available")
    return p


def test_oracle_under_sanitizers(tmp):
    exe = tmp / "oracle_check"
    cmd = ["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
           os.path.join(HERE, "sanitize", "oracle_check.c"), "-o", str(exe), "-lm"]
    assert "oracle ok" in _build_and_run(cmd, exe, tmp)


def test_repack_under_sanitizers(tmp):
    exe = tmp / "repack_check"
    csrc = os.path.join(os.path.dirname(HERE), "bit_weight_gemm_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, os.path.join(HERE, "sanitize", "repack_check.cpp"),
           os.path.join(csrc, "repack.cpp"), "-o", str(exe)]
    assert "repack ok" in _build_and_run(cmd, exe, tmp)
