"""The public header is plain C99 and a C program linked against libkvq.so
can use the host-side entry points (built with gcc, run on the CPU)."""
import os
import shutil
import subprocess

import pytest

from query_agnostic_eviction_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_client(tmp_path):
    _lib.load()                       # refuses a missing or stale library
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = tmp_path / "abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"),
           "-L", libdir, "-lkvq", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True)
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True)
    assert out.returncode == 0, out.stdout
    assert out.stdout.strip().startswith("ok")
