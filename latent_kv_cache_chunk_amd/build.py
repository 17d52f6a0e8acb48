"""Build libmla_hip.so (the C-ABI library of HIP kernels) in-tree for gfx950.

    python -m latent_kv_cache_chunk_amd.build [--resource-usage]

Each .hip file under csrc/ is compiled with hipcc for gfx950 only, then all
objects are linked into latent_kv_cache_chunk_amd/libmla_hip.so.  Packed fp32
instructions are disabled for every device compilation.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_hip.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "append.hip", "absorb.hip", "attend.hip", "attend_wide.hip", "attend_mha.hip", "upproj.hip",
           "cache_ring.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla_hip.so)")


def common_flags(resource_usage: bool = False) -> list[str]:
    flags = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]
    if resource_usage:
        flags.append("-Rpass-analysis=kernel-resource-usage")
    return flags


def compile_one(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags(resource_usage)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: compile_one(s, resource_usage), SOURCES))
    for obj, out in results:
        if out and (verbose or resource_usage):
            print(out)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + [o for o, _ in results] + [f"--offload-arch={ARCH}", "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel VGPR/LDS/spill usage")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.resource_usage, args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
