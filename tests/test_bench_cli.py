"""bench.py's command line on the CPU: more than one GPU is refused with a message before
anything touches a GPU, and so are invalid step counts."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    out = run("--gpus", "2")
    assert out.returncode == 2
    assert "one GPU only" in out.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    out = run(env=env)
    assert out.returncode == 2 and "one GPU only" in out.stderr


def test_steps_must_be_positive():
    out = run("--steps", "0")
    assert out.returncode != 0 and "--steps" in out.stderr


def test_decode_step_workload():
    """The decode step of the bench line: max(1, T // 128) tokens close a window, every other
    token sits one position before its window's end, and the batch is the decode sweep's."""
    import numpy as np

    import synth
    _, pool = synth.config3_pool()
    for T in (1, 100, 1024):
        wl = synth.decode_step(T, state=pool)
        full = synth.config3(T, state=pool)
        act = wl.active_mask()
        assert int(act.sum()) == max(1, T // 128)
        assert np.array_equal(wl.positions[act], full.positions[act])
        assert np.array_equal(wl.positions[~act], full.positions[~act] - 1)
        assert np.all(wl.positions[~act] % 128 == 126)
