"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only).

The library is rebuilt with the sanitizers on its host code (hipcc
-Xarch_host -fsanitize=...; device code unchanged) and
tests/abi_sanitize_driver.c calls every entry point with invalid arguments:
each call must return an error status before any HIP call, with no
sanitizer report.  The pointers passed are host buffers, so the test runs
only where no GPU is visible (no /dev/kfd)."""
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-pointer argument checks run without a GPU")
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_abi_argument_checks_clean_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libq8gemm_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "int8_block_scaled_amd", "csrc", "*.hip")))
    build = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "int8_block_scaled_amd", "csrc"),
             *srcs, "-o", lib]
    subprocess.run(build, check=True, capture_output=True, text=True, timeout=900)
    exe = str(tmp_path / "abi_sanitize")
    link = [CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "abi_sanitize_driver.c"),
            lib, "-Wl,-rpath," + str(tmp_path), "-o", exe]
    subprocess.run(link, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
