"""CPU checks of bench.py's command line: it measures one GPU only, and says
so instead of running when asked for more (no GPU is touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_distributed_launch_is_refused_too():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "WORLD_SIZE 8" in r.stderr


def test_help_lists_the_options():
    r = _run(["--help"])
    assert r.returncode == 0
    for opt in ("--config", "--layout", "--banned", "--penalties", "--synthetic-rates", "--rollback"):
        assert opt in r.stdout
