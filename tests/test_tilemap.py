"""The matrix-core product's workgroup orders, on the host: the header
q8_tilemap.h (used by the kernels) compiled with g++ into a small checker
that enumerates tile grids and orders (tests/tilemap_check.cpp)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_block_scaled_amd", "csrc")


def test_workgroup_orders_are_bijections(tmp_path):
    exe = str(tmp_path / "tilemap_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I" + CSRC,
                    os.path.join(ROOT, "tests", "tilemap_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "failures 0" in out.stdout
