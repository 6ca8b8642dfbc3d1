"""Compile the HIP libraries for gfx950.

Every translation unit under csrc/ is compiled with hipcc in parallel and
linked into indexer_exact_top_amd/libitk.so, the product library exporting
the C ABI of include/itk.h.  The test-only probes under probe/ (include/
itk_probe.h) are linked into their own libitk_probe.so.  Packed-fp32 VALU
instructions are disabled for every kernel.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libitk.so")
PROBE_DIR = os.path.join(HERE, "probe")
PROBE_LIB_PATH = os.path.join(HERE, "libitk_probe.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("ITK_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    msgs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs[-40:]) + "\n")
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(path)} failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, path)


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip")))
    jobs = jobs or min(len(srcs) + len(probes), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + probes))
    _link(objs[:len(srcs)], LIB_PATH)
    _link(objs[len(srcs):], PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
