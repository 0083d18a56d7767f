"""Host builds under the address and undefined-behaviour sanitizers (any
report aborts): the library's argument validation and planning
(tests/host_check.cpp: layouts, work splits, kernel index ranges and the
unsupported sizes, over a grid of shapes past the supported limits) and the
C oracle with its edge cases (tests/oracle_check.c)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(exe):
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    return out.stdout


def test_plans_and_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-Wall", *SAN, os.path.join(HERE, "host_check.cpp"),
                           "-o", str(exe)])
    assert "plans ok" in _run(exe)


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_check"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-fopenmp", *SAN,
                           os.path.join(HERE, "oracle_check.c"), "-o", str(exe), "-lm"])
    assert "oracle ok" in _run(exe)
