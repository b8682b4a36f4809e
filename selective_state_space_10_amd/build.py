"""Build the HIP library ``libssm_scan.so`` in-tree with hipcc for gfx950.

Every source is compiled on each call (object files go to ``_build/``), then
linked into ``selective_state_space_10_amd/libssm_scan.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_scan.so")
ARCH = "gfx950"

SOURCES = ["ssm_api.cpp", "scan_fwd.hip", "scan_bwd.hip", "state_update.hip", "affine_scan.hip"]
# the vector-ALU rate probes (a measurement tool beside the library)
PROBE_SOURCES = ["alu_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libssm_alu_probe.so")

# Packed FP32 instructions are switched off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
