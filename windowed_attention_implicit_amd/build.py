"""Builds librib.so (the HIP library behind include/rib.h) in-tree for gfx950.

Usage: python -m windowed_attention_implicit_amd.build  (or build() from Python).
Every .hip file under csrc/ is compiled with hipcc for --offload-arch=gfx950
into _build/ at the repository root, then linked into
windowed_attention_implicit_amd/librib.so.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "librib.so")

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # no packed fp32 instructions: compile plain float code to scalar VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # per-kernel register / scratch report, checked below: no kernel of the library may spill
    # registers to scratch memory
    "-Rpass-analysis=kernel-resource-usage",
]
# Per-file extra flags. The backward kernels keep more live state than 256
# arch VGPRs; left to its heuristics the compiler then gives the score / dP
# MFMAs the AGPR form and copies every result back to VGPRs for the exp and
# the products (hundreds of v_accvgpr moves per tile). The VGPR form keeps the
# MFMA results where the vector code reads them.
FILE_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build librib.so")


def _scratch_kernels(remarks: str) -> list:
    """Kernels whose resource-usage remarks report scratch (per-lane stack memory): register
    spills to memory. Spills into the accumulation registers (AGPRs) use no memory and pass."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "remark: Function Name:" in line:
            name = line.split("Function Name:")[1].split("[-Rpass")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split("[-Rpass")[0].strip())
            if n:
                bad.append(f"{name} ({n} bytes per lane)")
    return bad


def _compile(hipcc: str, src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = proc.stdout + proc.stderr
    msgs = "\n".join(l for l in out.splitlines()
                     if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{msgs}")
    spills = _scratch_kernels(out)
    if spills:
        raise RuntimeError(f"{src}: kernels spill registers to scratch memory: " + "; ".join(spills))
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every csrc/*.hip and links librib.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, verbose), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"linking librib.so failed:\n{' '.join(cmd)}\n{proc.stdout}{proc.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
