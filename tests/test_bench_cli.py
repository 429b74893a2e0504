"""CPU checks of bench.py's command line: more than one GPU is refused with
exit status 2 and a message that says why (the library runs on one GPU),
before any device is touched."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="8", RANK="0", LOCAL_RANK="0")
    r = _bench("--gpus", "8", env=env)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_unknown_workload_is_an_argument_error():
    r = _bench("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr
