"""bench.py's command-line contract on the host (no GPU): more than one GPU is refused with a
message, and every workload name it accepts is one the generators define."""
import os
import subprocess
import sys

import pytest

from sliding_window_gqa_varlen_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_workload_choices_match_the_generators():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    text = "".join(r.stdout.split())
    for w in W.WORKLOADS + W.EXTRA_WORKLOADS:
        assert w.name in text
