"""The library's window and division helpers, checked on the host (no GPU):
compiles tests/host/geometry_check.cpp with hipcc and runs it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_geometry_helpers(tmp_path):
    exe = tmp_path / "geometry_check"
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "--offload-arch=gfx950",
                    os.path.join(HERE, "host", "geometry_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "geometry: ok" in r.stdout
