"""Build libsdm.so for gfx950 in-tree with hipcc.

    python -m sparse_memory_linear_pk_amd.build [--jobs N]

Each HIP source compiles to an object in parallel; the objects link into
sparse_memory_linear_pk_amd/libsdm.so.  Packed-FP32 instruction generation is
turned off for every device pass.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsdm.so")
SOURCES = ["sdm_scan.hip", "sdm_scan_staged.hip", "sdm_api.hip", "pk_score.hip", "pk_topk.hip", "hbm_pattern.hip", "sdm_step.hip",
           "sdm_backward.hip", "sdm_project.hip", "sdm_diag.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if noise.strip():
        sys.stderr.write(noise + "\n")
    return obj


def build(jobs: int = 4, extra=()) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    print(build(args.jobs))
