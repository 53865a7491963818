"""bench.py's command line (CPU): more than one GPU is refused with a message
and a nonzero status before any GPU work, and --help documents the options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120,
                          env={**os.environ, **(env or {})})


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE=4" in r.stderr


def test_help_lists_the_options():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--rotate", "--no-configs", "--no-percall", "--no-cpu-baseline",
                "--cpu-workers"):
        assert opt in r.stdout
