"""The checked build on the GPU (tests/checked_driver.py, in a process of its
own with ORR_CHECKED=1): oracle parity with no check firing on clean inputs,
and a corrupted leaf range reported by the walks as ORR_ERR_HIP."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_checked_build():
    env = dict(os.environ, ORR_CHECKED="1")
    print("[case] checked build driver", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "checked_driver.py")], env=env,
                       capture_output=True, text=True, timeout=110)
    print(r.stdout[-4000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0
    assert "checked driver ok" in r.stdout
