"""The C ABI from a C99 program (host-side behaviour only, no GPU needed).

Compiles tests/c_abi/abi_host.c with gcc against include/mla.h, links it to the
built libmla.so and runs it: the header is valid C, the library links and
loads without Python or torch, and the host-side checks hold.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_latent_kv_16_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_client(tmp_path):
    lib = os.path.join(PKG, "libmla.so")
    assert os.path.exists(lib), "libmla.so is not built"
    exe = tmp_path / "abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "abi_host.c"),
           "-o", str(exe), "-L", PKG, "-lmla", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
