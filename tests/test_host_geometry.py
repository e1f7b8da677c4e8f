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


def test_launch_shapes(tmp_path):
    """Every launch the planners lead to fits one dispatch (workgroups x
    threads < 2^32) and the launches of a kernel cover every tile once, up
    to 2^28 planes (tests/host/launch_check.cpp, built with plan.hip)."""
    exe = tmp_path / "launch_check"
    csrc = os.path.join(os.path.dirname(HERE), "bwd_max_pool3d_amd", "csrc")
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "--offload-arch=gfx950",
                        os.path.join(HERE, "host", "launch_check.cpp"),
                        os.path.join(csrc, "plan.hip"), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "launch: ok" in r.stdout
