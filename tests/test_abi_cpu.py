"""CPU checks of the C-ABI library: it loads, exports every function that
include/dsa_indexer.h declares, and rejects bad arguments before any GPU work."""
import ctypes
import os
import re

import pytest

import sparse_attention_token_indexer_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        from sparse_attention_token_indexer_amd import build
        build.build()
    return dsa.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("indexer_score_topk", "misa_route_score_topk", "hisa_block_filter_topk",
              "indexer_mean_pool_keys", "indexer_selection_iou", "dsa_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) <= set(dsa._SIGS)
    assert lib.dsa_abi_version() == 3


def test_workspace_sizes_are_positive_and_monotone(lib):
    a = dsa.indexer_score_topk_workspace_size(64, 64, 128, 64, 131072, 2048)
    b = dsa.indexer_score_topk_workspace_size(64, 64, 128, 64, 262144, 2048)
    assert 0 < a < b
    assert dsa.misa_route_score_topk_workspace_size(64, 64, 128, 64, 131072, 64, 8, 8192, 2048, 1) > a
    assert dsa.hisa_block_filter_topk_workspace_size(32, 32, 128, 32, 1 << 20, 128, 64, 2048, 1) > 0
    assert dsa.indexer_score_topk_workspace_size(0, 64, 128, 1, 100, 8) == 0


def _call_dense(lib, **kw):
    args = dict(q=8, w=8, k=8, dtype=0, q_seq=None, q_pos=8, nq=1, H=8, d=128, n_seq=1,
                l_max=100, top_k=4, out_idx=8, out_score=None, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    # fake pointers are never dereferenced: every case below fails validation first
    return lib.indexer_score_topk(*[args[x] for x in (
        "q", "w", "k", "dtype", "q_seq", "q_pos", "nq", "H", "d", "n_seq", "l_max", "top_k",
        "out_idx", "out_score", "ws", "ws_bytes", "stream")])


def test_argument_errors_return_before_any_launch(lib):
    aligned = 1 << 20
    assert _call_dense(lib, q=aligned, k=aligned, top_k=0) == 1
    assert b"top_k" in lib.dsa_last_error()
    assert _call_dense(lib, q=aligned, k=aligned, d=96) == 2
    assert _call_dense(lib, q=aligned, k=aligned, H=65) == 2
    assert _call_dense(lib, q=aligned, k=aligned, dtype=7) == 1
    assert _call_dense(lib, q=aligned + 2, k=aligned) == 1            # misaligned q
    assert _call_dense(lib, q=None, k=aligned) == 1                    # NULL q
    assert _call_dense(lib, q=aligned, k=aligned, ws_bytes=10) == 3    # workspace too small
    assert b"workspace" in lib.dsa_last_error()
    assert _call_dense(lib, nq=0) == 0                                 # nothing to do
    assert _call_dense(lib, q=aligned, k=aligned, l_max=8192 * 8192 + 1) == 2   # too long
    assert b"l_max" in lib.dsa_last_error()
    assert lib.indexer_mean_pool_keys(aligned, 1, 1, 100, 128, 64, aligned, None) == 2
    assert lib.indexer_selection_iou(aligned, aligned, 1, 9000, aligned, None) == 2
    assert lib.misa_route_score_topk(aligned, aligned, aligned, None, 0, None, aligned, 1, 8, 128,
                                     1, 100, 16, 9, 0, 4, aligned, None, None, None, None, None,
                                     0, None) == 1                   # h > n_heads
    assert lib.hisa_block_filter_topk(aligned, aligned, aligned, None, 1, None, aligned, 1, 8, 128,
                                      1, 100, 16, 4, 4, aligned, None, None, None, None, None,
                                      0, None) == 2                  # f32 HISA unsupported
    assert lib.hisa_block_filter_topk(aligned, aligned, aligned, None, 0, None, aligned, 1, 8, 128,
                                      1, 100, 16, 4, 4, aligned, None, None, None, aligned + 2,
                                      None, 0, None) == 1            # misaligned out_status
    assert b"out_status" in lib.dsa_last_error()


def _call_mla(lib, **kw):
    args = dict(q=16, kv=16, dtype=0, q_seq=None, q_pos=4, idx=4, nq=2, H=32, d_qk=576, d_v=512,
                n_seq=1, l_max=100, top_k=256, scale=0.1, out=16, ws=None, ws_bytes=0,
                stream=None)
    args.update(kw)
    # fake pointers are never dereferenced: every case below fails validation first
    return lib.sparse_mla_attention(*[args[x] for x in (
        "q", "kv", "dtype", "q_seq", "q_pos", "idx", "nq", "H", "d_qk", "d_v", "n_seq", "l_max",
        "top_k", "scale", "out", "ws", "ws_bytes", "stream")])


def test_sparse_attention_rejects_bad_arguments(lib):
    EINVAL, EUNSUP, EWS = 1, 2, 3
    assert _call_mla(lib, dtype=1) == EUNSUP
    assert _call_mla(lib, d_qk=512) == EUNSUP
    assert _call_mla(lib, d_v=576) == EUNSUP
    for H in (16, 48, 160):
        assert _call_mla(lib, H=H) == EUNSUP
    assert _call_mla(lib, top_k=0) == EUNSUP
    assert _call_mla(lib, top_k=32769) == EUNSUP
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert _call_mla(lib, scale=s) == EINVAL
    assert _call_mla(lib, nq=-1) == EINVAL
    assert _call_mla(lib, q=None) == EINVAL
    assert _call_mla(lib, q=8) == EINVAL               # not 16-byte aligned
    assert _call_mla(lib, idx=2) == EINVAL             # not 4-byte aligned
    assert _call_mla(lib) == EWS                       # two queries: the lists are split
    assert _call_mla(lib, nq=0, q=None, kv=None, out=None) == 0


def test_sparse_attention_workspace_sizes(lib):
    # 64 queries x 128 heads x 2048 rows: two 64-head workgroups per (query,
    # slice), so 2 slices of 32 steps fill 256 compute units; bf16 slice
    # outputs and (reference, sum) pairs
    n = dsa.sparse_mla_workspace_size(64, 128, 576, 512, 2048)
    assert n == 64 * 2 * 128 * 512 * 2 + 64 * 2 * 128 * 8
    assert dsa.sparse_mla_workspace_size(256, 128, 576, 512, 2048) == 0   # one slice each
    assert dsa.sparse_mla_workspace_size(2, 32, 576, 512, 16) == 0        # one step
    assert dsa.sparse_mla_workspace_size(2, 32, 576, 512, 32769) == 0     # unsupported


def _call_misa_hisa(lib, **kw):
    args = dict(q=16, w=4, k=16, kp=None, dtype=0, q_seq=None, q_pos=4, nq=1, H=32, d=128,
                n_seq=1, l_max=4096, B=128, h=8, m=16, top_k=64, out_idx=4, out_score=None,
                heads=None, imp=None, blocks=None, bscore=None, status=None, ws=None, ws_bytes=0,
                stream=None)
    args.update(kw)
    return lib.misa_hisa_topk(*[args[x] for x in (
        "q", "w", "k", "kp", "dtype", "q_seq", "q_pos", "nq", "H", "d", "n_seq", "l_max", "B",
        "h", "m", "top_k", "out_idx", "out_score", "heads", "imp", "blocks", "bscore", "status",
        "ws", "ws_bytes", "stream")])


def test_misa_hisa_rejects_bad_arguments(lib):
    EINVAL, EUNSUP, EWS = 1, 2, 3
    assert _call_misa_hisa(lib, h=0) == EINVAL
    assert _call_misa_hisa(lib, h=33) == EINVAL
    assert _call_misa_hisa(lib, m=0) == EINVAL
    assert _call_misa_hisa(lib, B=0) == EINVAL
    assert _call_misa_hisa(lib, dtype=1) == EUNSUP
    assert _call_misa_hisa(lib, m=65, B=128) == EUNSUP       # m * B above 8192
    assert _call_misa_hisa(lib, m=1025, B=4) == EUNSUP       # more blocks than supported
    assert _call_misa_hisa(lib, status=6) == EINVAL          # misaligned out_status
    assert _call_misa_hisa(lib) == EWS
    assert dsa.misa_hisa_topk_workspace_size(32, 32, 128, 32, 1 << 20, 128, 8, 64, 2048, 1) > \
        dsa.hisa_block_filter_topk_workspace_size(32, 32, 128, 32, 1 << 20, 128, 64, 2048, 1)


def test_hisa_wait_limit_hook(lib):
    """The test hook that bounds the HISA token pass's wait is callable without a
    GPU (it only sets the limit later calls pass to the kernel)."""
    assert lib.dsa_hisa_wait_limit(0) == 0
    assert lib.dsa_hisa_wait_limit(-1) == 0          # back to the default
    assert lib.dsa_abi_version() == 3


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_device_work(lib):
    """The no-allocation dense entry point checks the call's workspace need
    against its fixed per-GPU scratch before it touches the device."""
    aligned = 1 << 20
    args = [aligned, aligned, aligned, 0, None, aligned, 64, 64, 128, 64, 1 << 21, 2048, aligned,
            None, None]
    assert lib.indexer_score_topk_noalloc(*args) == 2           # 64 x 2M keys: too large
    assert b"scratch" in lib.dsa_last_error()
    args[11] = 0
    assert lib.indexer_score_topk_noalloc(*args) == 1           # top_k 0
    assert dsa.indexer_score_topk_workspace_size(64, 64, 128, 64, 131072, 2048) <= \
        dsa.NOALLOC_SCRATCH_BYTES                                 # the dense decode workload fits
