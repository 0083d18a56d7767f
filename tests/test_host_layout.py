"""Host build of the MFMA tile-geometry checks (tests/layout_check.cpp)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_mfma_tile_layout(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-Wall", "-fsanitize=address,undefined",
                           os.path.join(HERE, "layout_check.cpp"), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "layout ok" in out.stdout
