"""bench.py's argument handling, on the host: the refusals that come before
any device use."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_reason():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_only_is_refused_outside_the_verify_workload():
    r = run("--config", "1", "--only", "step_m")
    assert r.returncode == 2
    assert "--only applies to --config 2" in r.stderr and r.stdout == ""


def test_unknown_workload_is_refused():
    r = run("--config", "99")
    assert r.returncode == 2 and r.stdout == ""
