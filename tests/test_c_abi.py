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


ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime.h")),
                    reason="HIP headers not available")
def test_planner_under_sanitizers(tmp_path):
    """The host planner built with g++ under ASan + UBSan, driven by
    tests/c_abi/plan_host.cpp: argument errors, capacity errors with exactly
    sized buffers, edge and random length mixes, the plan's invariants."""
    exe = tmp_path / "plan_host"
    csrc = os.path.join(PKG, "csrc")
    # host code only: the planner source and the driver, no device code
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", csrc, os.path.join(ROOT, "tests", "c_abi", "plan_host.cpp"),
           os.path.join(csrc, "plan.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    # a library preloaded by the environment would otherwise make ASan refuse to start
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
