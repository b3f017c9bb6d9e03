"""The bench's command line on the host: one GPU only, refused before any
device work (the bench measures the round on a single MI355X)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=e,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "requested 2" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused_too():
    r = _bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_workloads_and_protocol_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--steps", "--warmup", "--repeats", "--cpu-rows", "--layers", "--live-mask"):
        assert opt in r.stdout
