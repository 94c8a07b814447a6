"""Builds the sanitizer drivers of tests/test_sanitizers.py (CPU only).

oracle_checks: the C oracle (sdm_oracle*.c) with gcc -fsanitize=address,undefined.
host_checks:   the library's HIP sources with the host pass instrumented
               (-Xarch_host before each -fsanitize=; the device pass is built at
               -O0 only to link, it never runs), linked with the C driver.
Outputs go to tests/sanitize/_build/; each is rebuilt when a source is newer.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ORACLE = os.path.join(ROOT, "oracle")
CSRC = os.path.join(ROOT, "sparse_memory_linear_pk_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "_build")
HIP_SOURCES = ["sdm_scan.hip", "sdm_scan_staged.hip", "sdm_api.hip", "pk_score.hip", "pk_topk.hip",
               "hbm_pattern.hip", "sdm_step.hip", "sdm_backward.hip", "sdm_project.hip", "sdm_diag.hip"]
ORACLE_SOURCES = ["sdm_oracle.c", "sdm_oracle_grad.c", "sdm_oracle_proj.c", "sdm_oracle_diag.c"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
            "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _stale(target, sources):
    return not os.path.exists(target) or os.path.getmtime(target) < max(os.path.getmtime(s) for s in sources)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr[-4000:]}")


def oracle_checks() -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_checks")
    srcs = [os.path.join(HERE, "oracle_checks.c")] + [os.path.join(ORACLE, s) for s in ORACLE_SOURCES]
    if _stale(exe, srcs + [os.path.join(ORACLE, h) for h in os.listdir(ORACLE) if h.endswith(".h")]):
        _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-ffp-contract=off", "-I", ORACLE, *srcs, "-o", exe, "-lm"])
    return exe


def host_checks(jobs: int = 8) -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_checks")
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + [os.path.join(INCLUDE, "sdm.h")]
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    driver = os.path.join(HERE, "host_checks.c")
    if not _stale(exe, srcs + hdrs + [driver]):
        return exe

    def compile_one(src):
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        _run(["hipcc", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-O1", "-g", "-Xarch_device", "-O0",
              *HOST_SAN, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC,
              "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(OUT, "host_checks_main.o")
    _run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-I", INCLUDE, "-c", driver, "-o", drv])
    _run(["hipcc", "--offload-arch=gfx950", *HOST_SAN, drv, *objs, "-o", exe])
    return exe


if __name__ == "__main__":
    print(oracle_checks())
    print(host_checks())
