"""CPU checks of bench.py's command line: one GPU only (a request for more
exits with status 2 and says so, before touching torch or the GPU), and the
modes the measurement reports are produced with are all accepted."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_help_lists_every_mode():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--no-cpu-baseline", "--sweep", "--configs",
                 "--ceiling", "--copy-calibration"):
        assert flag in r.stdout
