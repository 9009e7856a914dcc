"""The C ABI from a plain C program (host-only calls; no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fp8_block_scaled_grouped_amd")


def test_c_consumer_links_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.exists(os.path.join(LIBDIR, "libmoe355.so")):
        pytest.skip("no C compiler or libmoe355.so not built")
    exe = str(tmp_path / "abi_consumer")
    cmd = [cc, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I/opt/rocm/include", os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", exe,
           "-L" + LIBDIR, "-lmoe355", "-Wl,-rpath," + LIBDIR]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
