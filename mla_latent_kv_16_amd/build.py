"""Compile libmla.so for gfx950 with hipcc (runs on a CPU-only host too).

    python -m mla_latent_kv_16_amd.build          # build into the package directory
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "libmla")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# Sources whose kernels get their leading arguments preloaded into SGPRs at
# wave launch (gfx950 kernel-argument preload; the compiler adds the fallback
# prologue that loads them from memory).  Their kernels list first the
# arguments that the first memory accesses depend on, so that the dependent
# chain before the first cache-row load starts without a kernarg round trip.
PRELOAD_SOURCES = {"decode_fast.hip"}
PRELOAD_FLAGS = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# (SGPR spills go to VGPR lanes; they reach memory only through ScratchSize)
_REMARK = re.compile(r"remark: +(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill): +(\S+)")


def _check_resources(src: str, text: str) -> None:
    """Every kernel must keep its data in registers and LDS: a kernel that
    uses scratch (private memory), by a spill or a stack array the compiler
    could not promote, runs many times slower, so the build refuses it."""
    kernel, bad = None, []
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            kernel = val
        elif val != "0":
            bad.append(f"{kernel}: {key} {val}")
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory:\n  " + "\n  ".join(bad))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    is_hip = src.endswith(".hip")
    lang = ["-x", "hip"] if is_hip else []
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if is_hip else []
    preload = PRELOAD_FLAGS if os.path.basename(src) in PRELOAD_SOURCES else []
    cmd = ["hipcc", *HIPCC_FLAGS, *preload, *lang, *remarks, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    out = "\n".join(line for line in text.splitlines()
                    if "packed-fp32-ops" not in line       # the host pass does not know the feature
                    and "kernel-resource-usage" not in line and not line.startswith(" "))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if is_hip:
        _check_resources(src, text)
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    if shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found on PATH")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           f"-Wl,-rpath,{ROCM}/lib", "-Wl,-soname,libmla.so"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
