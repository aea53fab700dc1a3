"""The C ABI used from C: tests/c_client/fa2_c_client.c includes only
include/fa2.h, is compiled with gcc and linked against libfa2.so, and checks
the argument errors and launch description without a GPU (every call it makes
with pointers carries an error checked before any HIP call)."""
import os
import subprocess

import pytest

import attention_forward_fa2_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are passed only where no GPU exists")
def test_c_client(tmp_path):
    fa2.load_library()  # raises if the library has not been built
    lib_dir = os.path.dirname(fa2.LIB_PATH)
    exe = str(tmp_path / "fa2_c_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_client", "fa2_c_client.c"), "-o", exe,
           "-L", lib_dir, "-l:libfa2.so", f"-Wl,-rpath,{lib_dir}"]
    subprocess.run(cmd, check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "C CLIENT OK" in out.stdout
