"""Q8_ERR_DEVICE, forced from the host: with every GPU hidden from the HIP
runtime (HIP_VISIBLE_DEVICES / ROCR_VISIBLE_DEVICES set to an invalid
index), every entry point given otherwise valid arguments must stop at its
device check and return Q8_ERR_DEVICE.  The calls run in a child process,
so this holds on a machine with a GPU too: nothing can be launched there."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def test_every_entry_point_reports_missing_device():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, os.path.join(HERE, "device_error_driver.py")],
                         env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "all entry points: Q8_ERR_DEVICE" in out.stdout
