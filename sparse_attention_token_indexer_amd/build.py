"""Build libdsa_indexer.so (gfx950) in-tree with hipcc.

``python -m sparse_attention_token_indexer_amd.build`` compiles every HIP source
under csrc/ for gfx950 and links the shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from typing import List

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libdsa_indexer.so")
SOURCES = ["api.hip", "k_score_select.hip", "k_prefill.hip", "k_prefill_routed.hip", "k_pool.hip",
           "k_route.hip", "k_hisa.hip", "k_mla.hip",
           "k_iou.hip", "k_certify.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd: List[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")


def build(jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJ, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
