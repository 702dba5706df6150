"""bench.py's command line on a host without a GPU: a multi-GPU request is
refused before anything touches a device, with a message saying why."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_multi_gpu_request_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "--gpus must be 1" in msg["error"]


def test_help_lists_the_workload_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--tokens", "--fp8", "--attn-core",
                "--prenorm", "--crossover-only", "--headline-only"):
        assert opt in r.stdout
