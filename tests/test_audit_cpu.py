"""Host-side bounds audit of every kernel launch (no GPU needed).

The library's C-ABI layer (csrc/api.hip: argument checks, workspace plans,
launch arguments) is compiled for the host with the address sanitizer and
linked with tests/audit/kernel_model.cpp, which replaces each kernel launch by
a walk over the kernel's grid that derives, from the kernel's own index
arithmetic, the byte range of every global-memory access.  tests/audit/drive.py
calls every entry point with fake device addresses of exactly sized buffers -
the full-size workloads (among them the HISA test's three calls at 32 queries
x 1048576 keys: HISA, the dense 32-head indexer and the IoU), a seeded sweep of
random shapes and positions (some invalid), and planted mistakes (one buffer
one element too small) that the audit must catch.
"""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_token_indexer_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "audit")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc",):
        if os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def audit_lib():
    os.makedirs(OUT, exist_ok=True)
    asan = _asan_runtime()
    lib = os.path.join(OUT, "libdsa_audit.so")
    san = ["-Xarch_host", "-fsanitize=address"] if asan else []
    common = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", *san]
    api_o = os.path.join(OUT, "api.o")
    model_o = os.path.join(OUT, "kernel_model.o")
    # api.hip with its device part (it defines the no-allocation entry point's
    # device array), the model for the host only (it replaces the kernels)
    steps = [
        [_hipcc(), "--offload-arch=gfx950", *common, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o],
        [_hipcc(), "-x", "hip", "--cuda-host-only", *common, "-c",
         os.path.join(ROOT, "tests", "audit", "kernel_model.cpp"), "-o", model_o],
        [_hipcc(), "--offload-arch=gfx950", "-shared", *san, api_o, model_o, "-o", lib],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr
    return lib, asan


def test_every_kernel_access_stays_inside_its_buffers(audit_lib):
    lib, asan = audit_lib
    env = dict(os.environ)
    if asan:
        env["LD_PRELOAD"] = asan
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "audit", "drive.py"), lib, "150"],
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.stdout.strip(), r.stderr[-4000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print(f"audit: {res['cases']} calls, launches {res['launches']}")
    assert not res["violations"], "\n".join(res["violations"][:10])
    assert not res["planted_missed"], res["planted_missed"]
    assert r.returncode == 0, r.stderr[-4000:]
    # every kernel of the library was modelled at least once
    for k in ("k_score_emit", "k_score_emit(store_all)", "k_merge", "k_select_short", "k_prepare",
              "k_mean_pool", "k_route", "k_route_rows", "k_route_prefill", "k_route_heads",
              "k_pool_prefix", "k_prefill_score", "k_prefill_routed_score", "k_prefill_select",
              "k_hisa", "k_iou", "k_sparse_mla", "k_certify_heads", "k_certify_compact"):
        assert res["launches"].get(k, 0) > 0, k
