"""The 3-bit codec's decision table (q8_kv3_table.h, used by the encode
kernel) against the oracle's rule on every binary32 input: the code of u
must be the number of thresholds t_k <= u, the thresholds being the
binary32 midpoints of the oracle's Lloyd-Max levels (signalling NaNs, which
no arithmetic produces, excepted)."""
import os
import subprocess

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_block_scaled_amd", "csrc")


def test_code_table_matches_oracle_rule_exhaustively(orc, tmp_path):
    L = orc.kv3_levels()
    t = ((L[:-1] + L[1:]) * np.float32(0.5)).astype(np.float32)   # binary32 midpoints
    assert np.all(np.diff(t) > 0)
    exe = str(tmp_path / "kv3_table_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-fopenmp", "-I" + CSRC,
                    os.path.join(ROOT, "tests", "kv3_table_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe] + ["%08x" % b for b in t.view(np.uint32)], capture_output=True,
                         text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert ": 0 mismatches" in out.stdout
