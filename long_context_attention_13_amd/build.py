"""Build liblca.so (gfx950 only) in-tree with hipcc.

Every HIP translation unit under csrc/ is compiled for gfx950 with packed
fp32 vector ops disabled, then linked with the C-ABI layer into one shared
library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblca.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]

SOURCES = ["compress.hip", "index.hip", "index_prefill.hip", "attend.hip", "attend_dense.hip", "step.hip", "append.hip", "noalloc.hip", "abi.cpp"]
# per-source flags: keep MFMA results in ordinary VGPRs (the score kernel's
# epilogue reads every result; accumulation-register copies would double it)
EXTRA = {"index_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "step.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l
                     and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
