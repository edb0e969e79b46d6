"""bench.py's command line, on the CPU: the one-GPU guard and the options the
profiles' commands use (no GPU work is started)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120,
                          env=env, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_exits_too():
    env = dict(os.environ, WORLD_SIZE="2")
    r = run(env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_profile_options():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--no-cpu", "--no-context", "--calibrate", "--sustain", "--shape",
                "--shape-reps", "--shape-warmup", "--shape-rounds", "--traffic-probe"):
        assert opt in r.stdout, opt
