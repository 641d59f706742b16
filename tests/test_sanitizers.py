"""Host sanitizer builds (CPU only): the oracle and the library's host
relayout compiled with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc / g++, host code only; no device code is involved) and run through the
drivers in tests/sanitize/.  Any out-of-bounds access, leak, signed overflow
or other undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _run(cmd, tmp_path, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True, cwd=ROOT)
    # (verify_asan_link_order=0: a library preloaded by the environment may
    # come before the sanitizer runtime; the checks work either way)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(tmp_path / exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "oracle/iqk_oracle.c", "tests/sanitize/oracle_driver.c",
          "-o", str(exe), "-lm"], tmp_path, "oracle_san")


def test_host_relayout_under_sanitizers(tmp_path):
    exe = tmp_path / "relayout_san"
    csrc = "dequant_iqk_moe_amd/csrc/"
    _run(["g++", "-std=c++17", *SAN, "-pthread", csrc + "iqk_relayout.cpp", csrc + "iqk_status.cpp",
          "tests/sanitize/relayout_driver.cpp", "-o", str(exe)], tmp_path, "relayout_san")
