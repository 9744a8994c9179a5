"""bench.py's command-line contract, checked on the CPU (no GPU is touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = run_bench(env=env)
    assert r.returncode == 2
    assert r.stdout == ""


def test_help_lists_the_contract_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--only"):
        assert flag in r.stdout
