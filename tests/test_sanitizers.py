"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the fp64 oracle and
the C++ block manager, each built with gcc/g++ into a driver of its own (they share no binary)
and run on small random inputs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd_build, exe):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe], exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_manager_under_sanitizers(tmp_path):
    exe = str(tmp_path / "blocks_san")
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "sanitize", "blocks_driver.cpp"),
          os.path.join(ROOT, "paged_kv_cache_16_amd", "csrc", "blocks.cpp"), "-o", exe], exe)
