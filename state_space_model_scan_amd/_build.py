"""Builds libssmscan.so in-tree with hipcc for gfx950 (MI355X).

Every HIP source is compiled with the packed-FP32 feature switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``): hipcc then emits only
scalar fp32 VALU instructions.  hipcc's host pass warns that it does not know
the feature; that warning is harmless.  ``-mllvm -amdgpu-mfma-vgpr-form``
keeps matrix-core results in ordinary VGPRs, so the VALU reads them without
an accumulator-register copy.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssmscan.so")
# instruction-rate and bandwidth probes (bench.py --microbench), a library of
# their own so that the operator's ABI holds only the operator
MICRO_LIB = os.path.join(PKG, "libssmmicro.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", "-Wall"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-gpu-rdc"]

SOURCES = [
    ("scan_bf16.hip", True),
    ("scan_f32.hip", True),
    ("scan_f16.hip", True),
    ("scan_bf16_ew.hip", True),
    ("scan_f32_ew.hip", True),
    ("scan_f16_ew.hip", True),
    ("ssm_scan.hip", True),
    ("scan_complex.hip", True),
    ("decode.hip", True),
    ("ssd.hip", True),
    ("bwd.hip", True),
    ("bwd_complex.hip", True),
    ("validate.cpp", False),
]
MICRO_SOURCES = [("microbench.hip", True)]


def _compile(src: str, is_hip: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + (HIP_FLAGS if is_hip else ["-x", "c++"]) + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"linking {os.path.basename(lib)} failed")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libssmscan.so and libssmmicro.so (always
    rebuilds)."""
    srcs = SOURCES + MICRO_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(*s), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], MICRO_LIB)
    if verbose:
        print(f"built {LIB} and {MICRO_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
