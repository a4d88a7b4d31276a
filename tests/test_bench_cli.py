"""bench.py's command-line contract that can be checked without a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a refused run


def test_only_modes_are_listed_in_the_usage():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for mode in ("fwd", "fwd_causal", "fwd_4k", "fwd_gqa", "fwd_fp8", "bwd", "prefill_paged",
                 "decode", "copy"):
        assert mode in r.stdout
