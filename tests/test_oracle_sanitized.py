"""Sanitizer runs of the C test infrastructure (gcc, host code only, AddressSanitizer and
UndefinedBehaviorSanitizer).

The CPU oracle (oracle/c128_oracle.c), driven by tests/oracle_driver.c through the four cache
formats (C128, C4, indexer FP8, indexer MXFP4) and every early exit: a non-boundary position, a
negative state slot, an out-of-range request, an out-of-range block id, a negative and an
out-of-range kv slot.  The run must be free of memory errors, undefined behaviour and leaks,
give each token its expected status and leave every other cache byte unchanged.  Then the seeded
input generator (synth/synth_gen.c), driven by tests/synth_driver.c."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_driver"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "tests", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "c128_oracle.c"), "-lm", "-lpthread",
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert out.stdout.strip() == "oracle driver ok"


def test_input_generator_under_sanitizers(tmp_path):
    """The seeded input generator (synth/synth_gen.c) under the same sanitizers, driven by
    tests/synth_driver.c: a padded pool filled with 1 and with 5 threads gives identical values
    and leaves every padding element alone; the other fill functions stay inside their
    outputs."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "synth_driver"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "tests", "synth_driver.c"),
                    os.path.join(ROOT, "synth", "synth_gen.c"), "-lm", "-lpthread",
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert out.stdout.strip() == "synth driver ok"


@pytest.mark.parametrize("driver,sources", [
    ("oracle_driver.c", [os.path.join("oracle", "c128_oracle.c")]),
    ("synth_driver.c", [os.path.join("synth", "synth_gen.c")])])
def test_threads_under_thread_sanitizer(driver, sources, tmp_path):
    """Both C modules split their work over pthreads (the oracle by token, the generator by
    block); under ThreadSanitizer the same drivers run without a data race."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / (driver[:-2] + "_tsan")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=thread",
                    os.path.join(ROOT, "tests", driver),
                    *[os.path.join(ROOT, s) for s in sources], "-lm", "-lpthread",
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert "ThreadSanitizer" not in out.stderr
