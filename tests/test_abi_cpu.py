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
    assert lib.dsa_abi_version() == 1


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
                                      1, 100, 16, 4, 4, aligned, None, None, None, None, 0,
                                      None) == 2                     # f32 HISA unsupported
