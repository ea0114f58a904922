"""The no-allocation dense entry point (the library's per-GPU scratch instead
of a workspace) against indexer_score_topk: identical selections and scores on
two calls in a row, the second with a smaller input, and the oracle on sampled
rows.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import datagen
from oracle import indexer as O
from oracle.check import check_selection

from _helpers import say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_indexer_amd as m
    m.lib()
    return m


def _sorted_pairs(idx, val):
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    o = np.argsort(idx, axis=1, kind="stable")
    return np.take_along_axis(idx, o, 1), np.take_along_axis(val, o, 1)


def test_noalloc_matches_the_workspace_entry_point(dsa):
    errs = []
    for nq, L, H, k in ((16, 40000, 64, 1024), (5, 3000, 32, 2048)):   # second call smaller
        wl = datagen.small(2, nq=nq, n_seq=nq, l_max=L, n_heads=H)
        inp = datagen.make(wl, nq)
        dev = upload(inp, wl)
        say(f"[noalloc] nq={nq} L={L} H={H} k={k}")
        a_i, a_s = dsa.indexer_score_topk_noalloc(dev["q"], dev["w"], dev["k"], dev["q_pos"],
                                                  dev["q_seq"], top_k=k)
        b_i, b_s = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"],
                                          dev["q_seq"], top_k=k)
        torch.cuda.synchronize()
        ai, av = _sorted_pairs(a_i, a_s)
        bi, bv = _sorted_pairs(b_i, b_s)
        assert np.array_equal(ai, bi), f"nq={nq}: selections differ"
        assert np.array_equal(av, bv), f"nq={nq}: scores differ"
        for t in (0, nq - 1):
            q_t, w_t = O.to_f64(inp["q"][t], wl.dtype), inp["w"][t].astype(np.float64)
            K = O.to_f64(inp["k"][t], wl.dtype)
            r = O.dense_row(q_t, w_t, K, int(inp["q_pos"][t]), k)
            errs += check_selection(a_i[t].cpu().numpy(), a_s[t].cpu().numpy(), r["cand"], r["s"],
                                    r["A"], k, O.dot_magnitude(q_t, w_t, K[r["cand"]]),
                                    what=f"noalloc nq={nq} q{t}")
    assert not errs, "\n".join(errs[:8])
