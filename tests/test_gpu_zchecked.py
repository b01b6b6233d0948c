"""The checked library: every mode runs with the kernels' index-range checks
on and records no failed check, and a failed check is recorded (see
tests/checked_run.py, run in a process of its own)."""
import os
import subprocess
import sys

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_checked_library_records_no_failed_check():
    lib = os.path.join(os.path.dirname(HERE), "volume_rendering_amd", "libnerf_mi355x_checked.so")
    assert os.path.exists(lib), "build the checked library: python -m volume_rendering_amd.build"
    say("checked library run")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "checked_run.py")], capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-4000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
