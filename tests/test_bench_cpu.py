"""bench.py's command-line contract on a machine without a GPU: a request for
more than one GPU is refused with a message before torch or the library is
touched (the library has no multi-GPU path)."""
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "measures one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that was not measured
