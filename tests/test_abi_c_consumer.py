"""The boundary from plain C: tests/abi_consumer.c includes the public header, links against
the library with gcc (no Python or torch in between) and checks the host-only entry points
(validation error codes, workspace sizes, the version and the error message).  The same file
also compiles as C++, so the header's extern "C" block is exercised too."""

import os
import shutil
import subprocess

import pytest

import paged_kv_cache_fp32_amd as c128

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "abi_consumer.c")
INCLUDE = os.path.join(ROOT, "include")


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_c_consumer(lang, tmp_path):
    compiler = "gcc" if lang == "c" else "g++"
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    c128.library()  # raises if the library has not been built
    lib_dir = os.path.dirname(c128.LIBRARY_PATH)
    std = "-std=c11" if lang == "c" else "-std=c++17"
    exe = tmp_path / f"abi_consumer_{lang.replace('+', 'p')}"
    cmd = [compiler, "-x", lang, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE,
           SRC, "-x", "none", f"-L{lib_dir}", "-ldsv4_c128", f"-Wl,-rpath,{lib_dir}",
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "abi consumer ok"


def test_c_consumer_under_address_sanitizer(tmp_path):
    """The host validation code (c128_abi.cpp) built with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host pass only (-Xarch_host before each -fsanitize: no GPU
    code is instrumented) and linked into the plain C consumer, the kernels' launchers coming
    from the built library: every validation path the consumer drives, the stride-span guards
    against 64-bit overflow included, runs without an out-of-bounds access, a use after free or
    undefined behaviour."""
    hipcc = "/opt/rocm/bin/hipcc"
    if shutil.which("gcc") is None or not os.path.exists(hipcc):
        pytest.skip("gcc or hipcc not found")
    c128.library()
    lib_dir = os.path.dirname(c128.LIBRARY_PATH)
    csrc = os.path.join(ROOT, "paged_kv_cache_fp32_amd", "csrc")
    abi_o, cons_o, exe = tmp_path / "abi.o", tmp_path / "consumer.o", tmp_path / "consumer_asan"
    subprocess.run([hipcc, "-std=c++17", "-O1", "-g", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", csrc, "-c",
                    os.path.join(csrc, "c128_abi.cpp"), "-o", str(abi_o)],
                   check=True, capture_output=True, text=True)
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address", "-I", INCLUDE, "-c", SRC,
                    "-o", str(cons_o)], check=True, capture_output=True, text=True)
    subprocess.run(["g++", "-fsanitize=address,undefined", str(cons_o), str(abi_o), f"-L{lib_dir}",
                    "-ldsv4_c128", "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{lib_dir}",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert out.stdout.strip() == "abi consumer ok"
    assert "AddressSanitizer" not in out.stderr
