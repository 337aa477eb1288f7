"""Build the HIP library (libfa_mi355x.so) in-tree for gfx950.

Each translation unit under ``csrc/`` is compiled with hipcc into ``_build/`` in
parallel, then linked into ``exact_attention_fa_amd/libfa_mi355x.so``.  Usage:

    python -m exact_attention_fa_amd._build [--resource-usage]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_f32.hip", "fa_noalloc.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # Packed fp32 VALU forms are disabled for all device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


# Per-source device-code options.  MFMA results that feed VALU work (scores, dP) are wanted in
# VGPRs, which the VALU reads directly, not in AGPRs, which it cannot: the compiler chooses the
# AGPR form for every MFMA of a kernel that may use more than 256 VGPRs, so the VGPR form is
# forced (measured: dK/dV pass 6% fewer cycles; no other kernel changes).  The forward's MFMAs
# that accumulate in AGPRs are written as inline assembly.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
DEVICE_FLAGS = {"fa_bwd.hip": VGPR_FORM, "fa_fwd.hip": VGPR_FORM}


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), *DEVICE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(line for line in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{log}")
    return obj, log


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link the shared library; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    logs = [log for _, log in results if log.strip()]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose or resource_usage:
        for log in logs:
            print(log)
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/AGPR/LDS/scratch use from the compiler")
    args = ap.parse_args()
    path = build(resource_usage=args.resource_usage, verbose=True)
    print(path, file=sys.stderr)
