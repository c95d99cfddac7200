"""The C ABI from C: compile tests/c/abi_host_check.c as C99 with gcc against
include/sdpa_attn.h, link the built library and run it (host-only calls; no
GPU needed)."""
import os
import shutil
import subprocess

import pytest

from scaled_dot_product_15_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(binding.LIB_PATH) or shutil.which("gcc") is None,
                    reason="needs gcc and the built library")
def test_header_is_c_and_host_calls_work(tmp_path):
    exe = tmp_path / "abi_host_check"
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", str(exe), "-L", libdir,
           "-l:" + os.path.basename(binding.LIB_PATH), "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr
