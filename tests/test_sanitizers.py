"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
run without a GPU:

* the C-ABI layer (invariant_rmsnorm_amd/csrc/api.cpp) linked with host-only
  stand-ins for the kernel launchers (tests/sanitize/launch_stub.cpp, which
  check what the launchers rely on), driven over ordinary and extreme
  arguments by tests/sanitize/api_cases.cpp;
* the CPU oracle (oracle/rmsnorm_oracle.cpp) driven over every entry point
  by tests/sanitize/oracle_cases.cpp.

Both are built with g++ (host code only; nothing here is GPU code) and must
exit 0 with no sanitizer report."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ROOT / "tests" / "sanitize"
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build_and_run(tmp_path, name, sources, includes, extra=()):
    exe = tmp_path / name
    cmd = ["g++", *FLAGS, *extra, *(f"-I{i}" for i in includes), *map(str, sources), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    return report


def test_api_host_checks_under_sanitizers(tmp_path):
    csrc = ROOT / "invariant_rmsnorm_amd" / "csrc"
    out = _build_and_run(tmp_path, "api_cases",
                         [csrc / "api.cpp", SAN / "launch_stub.cpp", SAN / "api_cases.cpp"],
                         [ROOT / "include", csrc])
    assert "0 failures" in out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "oracle_cases",
                         [ROOT / "oracle" / "rmsnorm_oracle.cpp", SAN / "oracle_cases.cpp"],
                         [ROOT / "oracle"], extra=("-ffp-contract=off",))
    assert "0 failures" in out
