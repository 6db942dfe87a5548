"""The C header compiles as plain C99 and a C client linked against
libduoattn.so gets the documented results from the host-only entry points
(no GPU needed)."""
import os
import shutil
import subprocess

import pytest

import gqa_sliding_window_amd as g

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_client(lib, tmp_path):
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(g.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", f"-I{ROOT}/include",
           os.path.join(HERE, "c", "abi_check.c"), f"-L{libdir}", "-lduoattn", f"-Wl,-rpath,{libdir}", "-lm",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
