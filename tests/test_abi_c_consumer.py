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
