"""bench.py's command-line contract on the host (no GPU is touched): a run on
more than one GPU is refused with a message, and the argument defaults are
the ones the measurement description states."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "3", "--warmup", "1")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run("--steps", "3", env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_defaults():
    sys.path.insert(0, ROOT)
    import bench

    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert (a.gpus, a.steps, a.warmup, a.mode, a.workload) == (1, 320, 32, "eager", "llama8b_mxfp4")
    # The headline's algorithmic bytes: X once, codes and E8M0 scales once, T once.
    assert bench.algorithmic_bytes("mxfp4", 4096, 4096, 32) == 42729472
