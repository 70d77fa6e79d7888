"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the planner (pure host integer code) driven by a descriptor fuzzer, and the CPU
oracle driven by random small problems.  gcc / g++ build host code only here."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(cmd, exe, args=()):
    res = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    return run.stdout


def test_planner_under_asan_ubsan(tmp_path):
    out = _build_and_run(["g++", "-std=c++17", *SAN, os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp"),
                          os.path.join(ROOT, "implicit_gemm_amd", "csrc", "plan.cpp")],
                         str(tmp_path / "plan_fuzz"), ["1000000"])
    assert "0 failures" in out, out


def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(["gcc", "-std=c99", "-fopenmp", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_asan.c"),
                          os.path.join(ROOT, "oracle", "wgrad_ref.c"), "-lm"],
                         str(tmp_path / "oracle_asan"))
    assert "problems" in out, out
