"""Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two CPU programs, each built here with the GNU compilers and run:

* ``tests/native/plan_check.cpp`` with the library's host logic -- the
  launch planners (``pa_plan.cpp``) and the block manager
  (``pa_manager.cpp``) -- checking the planners' invariants on seeded
  random batches and at their limits (every non-empty (sequence,
  partition) listed once, merge rows exactly the multi-partition
  sequences, the launch order, the partition choice within the workspace,
  prefill tiles grouped and ordered, split slots disjoint and inside the
  workspace) and the manager on random programs;
* ``tests/native/oracle_check.c`` with the oracle (``oracle/oracle.c``),
  every entry point and error path on seeded random shapes.

The two programs share nothing: the oracle and the library's host code are
never linked together.  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "paged_kv_cache_05_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def build(tmp_path, name, cmd):
    out = str(tmp_path / name)
    res = subprocess.run(cmd + ["-o", out], capture_output=True, text=True)
    assert res.returncode == 0, f"build of {name} failed:\n{' '.join(cmd)}\n{res.stderr}"
    return out


def run(exe, *args):
    res = subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=600)
    assert res.returncode == 0, f"{exe} failed ({res.returncode}):\n{res.stdout}\n{res.stderr}"
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    return res.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planners_and_manager_sanitized(tmp_path):
    exe = build(tmp_path, "plan_check",
                ["g++", "-std=c++17", "-Wall", *SAN, "-I", CSRC, "-I",
                 os.path.join(ROOT, "include"), os.path.join(NATIVE, "plan_check.cpp"),
                 os.path.join(CSRC, "pa_plan.cpp"), os.path.join(CSRC, "pa_manager.cpp")])
    for seed in ("1", "2"):
        assert "plan_check ok" in run(exe, seed)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_sanitized(tmp_path):
    exe = build(tmp_path, "oracle_check",
                ["gcc", "-std=c99", "-Wall", "-Wno-unknown-pragmas", *SAN,
                 os.path.join(NATIVE, "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                 "-lm"])
    for seed in ("1", "2"):
        assert "oracle_check ok" in run(exe, seed)
