"""Host-side checks of bench.py's command line (no GPU needed): the defaults
run one GPU with a bounded number of steps, and a request for more than one
GPU is refused with a message instead of being run."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_defaults_are_one_gpu_and_bounded_steps():
    sys.path.insert(0, ROOT)
    import bench

    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = old
    assert args.gpus == 1 and 1 <= args.steps <= 100 and 0 <= args.warmup <= 100
    assert args.accum == "exact"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                 # no JSON line for a configuration it does not run
