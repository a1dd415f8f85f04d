"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Two drivers are built with gcc/g++ and -fsanitize=address,undefined (with
-fno-sanitize-recover, so that any finding fails the run):
  * the fp64 oracle (oracle/mhla_oracle.c, without OpenMP): blockwise and
    brute-force rows agree on small geometries, bad arguments are rejected;
  * the library's host-side argument checks (csrc/mhla_check.hpp, the code
    behind mhla_validate, mhla_num_blocks, mhla_lb_init and the checks of every
    entry point), including sizes at the int limits.
No device code is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr
    assert res.stdout.strip().endswith("ok")


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99"] + SAN + ["-o", exe, os.path.join(HERE, "oracle_driver.c"),
                                      os.path.join(ROOT, "oracle", "mhla_oracle.c"), "-lm"], exe)


def test_host_checks_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "check_driver")
    _run(["g++", "-std=c++17"] + SAN + ["-I", os.path.join(ROOT, "include"), "-I",
                                        os.path.join(ROOT, "token_level_head_mhla_amd", "csrc"),
                                        "-o", exe, os.path.join(HERE, "check_driver.cpp")], exe)
