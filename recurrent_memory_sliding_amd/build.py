"""Builds libmaglev.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m recurrent_memory_sliding_amd.build

Every translation unit is compiled with hipcc for --offload-arch=gfx950 and
packed fp32 arithmetic disabled, then linked into one shared library next to
this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmaglev.so")
SOURCES = ["maglev_api.cpp", "profile.cpp", "path.hip", "mfma_gemm.hip", "mfma_attn.hip",
           "loss_decode.hip", "gated_mix.hip", "loss_head.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-x", "hip", "-std=c++17", "-O3", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Extra compiler options of single translation units. The attention kernels
# keep their MFMA results in VGPRs: left to its heuristics the allocator put
# the score accumulators of the dK/dV pass in AGPRs overlapping the dK/dV
# accumulators and moved 96 registers between the two files on every tile.
FILE_FLAGS = {"mfma_attn.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    # only the maglev_* C functions are exported (maglev.map)
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950",
           "-Wl,--version-script=" + os.path.join(CSRC, "maglev.map"), "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
