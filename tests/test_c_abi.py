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


CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address", "-fsanitize=undefined"]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not available")
def test_c_client_under_host_sanitizers(lib, tmp_path):
    """The host side of the C ABI (validation, planning, workspace and cache
    arithmetic) built with AddressSanitizer and UndefinedBehaviorSanitizer,
    linked with the library's kernel objects, and driven by the plain C
    client: no memory error and no undefined behaviour (any report aborts).
    Host code only: the device code of the kernels is not instrumented."""
    from gqa_sliding_window_amd import build as B
    objdir = os.path.join(os.path.dirname(g.LIB_PATH), "_build")
    kernels = [os.path.join(objdir, s.split(".")[0] + ".o") for s in B.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(k) for k in kernels):
        pytest.skip("kernel objects not built")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    api_o = tmp_path / "api_san.o"
    cmd = [B.hipcc(), "-x", "hip", f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
           *host_san, "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           f"-I{B.INCLUDE}", f"-I{B.CSRC}", "-c", os.path.join(B.CSRC, "api.cpp"), "-o", str(api_o)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    so = tmp_path / "libduoattn.so"
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", str(api_o), *kernels, "-o", str(so)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_check_san"
    cmd = [CLANG, "-std=c99", "-g", *SAN, "-fno-sanitize-recover=all", f"-I{ROOT}/include",
           os.path.join(HERE, "c", "abi_check.c"), f"-L{tmp_path}", "-lduoattn", f"-Wl,-rpath,{tmp_path}",
           "-lm", "-lstdc++", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-3000:]
