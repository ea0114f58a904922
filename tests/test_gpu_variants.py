"""GPU parity of MISA, MISA dagger and HISA against the CPU oracle.

Every stage is checked on its own, conditionally on the GPU's own upstream
choice: the routed heads against the oracle's importance, the coarse
candidates against the oracle's routed scores given those heads, the final
selection against the oracle's scores over the GPU's candidates.  A near-tie
upstream therefore cannot turn into a false failure downstream.
"""
import numpy as np
import pytest
import torch

import datagen
from oracle import indexer as O
from oracle.check import check_selection, scores_ok

from _helpers import say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_indexer_amd as m
    m.lib()
    return m


def _rows(inp, wl, t):
    s = int(inp["q_seq"][t])
    return (O.to_f64(inp["q"][t], wl.dtype), inp["w"][t].astype(np.float64),
            O.to_f64(inp["k"][s], wl.dtype), int(inp["q_pos"][t]))


def _check(gi, gv, cand, s, A, k, q_t, w_t, K, what, heads=None):
    qq, ww = (q_t, w_t) if heads is None else (q_t[heads], w_t[heads])
    F = O.dot_magnitude(qq, ww, K[cand]) if cand.size else np.zeros(0)
    return check_selection(gi, gv, cand, s, A, k, F, what=what)


def _misa_case(dsa, wl, h, k, kprime, seed=0, pos=None, pooled=True, rows=None):
    inp = datagen.make(wl, seed)
    if pos is not None:
        inp["q_pos"] = np.asarray(pos, dtype=np.int32)
    say(f"[misa] nq={wl.nq} L={wl.l_max} H={wl.n_heads} B={wl.block} h={h} k={k} k'={kprime} "
        f"pooled={pooled}")
    dev = upload(inp, wl)
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block) if pooled else None
    res = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    block=wl.block, n_active_heads=h, top_k=k, k_prime=kprime,
                                    k_pooled=kp, with_importance=True, with_cand=kprime > 0)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in res.items() if v is not None}
    errs = []
    for t in (range(wl.nq) if rows is None else rows):
        q_t, w_t, K, p = _rows(inp, wl, t)
        pooled_ref = O.misa_pooled_for_query(K, wl.block, p)
        I = O.misa_importance(q_t, w_t, pooled_ref)
        Fi = np.abs(w_t) * (np.abs(q_t) @ np.abs(pooled_ref).T).sum(axis=1)
        # router importance and head choice
        gi = out["importance"][t].astype(np.float64)
        bad = ~scores_ok(gi, I, I, Fi)
        if bad.any():
            errs.append(f"importance q{t}: heads {np.nonzero(bad)[0][:4]} gpu {gi[bad][:4]} ref {I[bad][:4]}")
        errs += check_selection(out["heads"][t], None, np.arange(wl.n_heads), I, I, h, Fi,
                                what=f"heads q{t}")
        heads = out["heads"][t].astype(np.int64)
        # routed pass, conditional on the GPU's heads
        r = O.misa_row(q_t, w_t, K, p, wl.block, h, kprime or k, heads=heads)
        if kprime == 0:
            errs += _check(out["idx"][t], out["score"][t], r["cand"], r["s"], r["A"], k,
                           q_t, w_t, K, f"misa q{t}", heads)
        else:
            errs += _check(out["cand"][t], None, r["cand"], r["s"], r["A"], kprime,
                           q_t, w_t, K, f"coarse q{t}", heads)
            f = O.rescore_row(q_t, w_t, K, out["cand"][t], k)
            errs += _check(out["idx"][t], out["score"][t], f["cand"], f["s"], f["A"], k,
                           q_t, w_t, K, f"dagger q{t}")
    assert not errs, "\n".join(errs[:12])
    return inp, out


def test_misa_reduced(dsa):
    wl = datagen.small(4, nq=8, n_seq=8, l_max=16384)
    _misa_case(dsa, wl, h=8, k=256, kprime=0)


def test_misa_dagger_reduced(dsa):
    wl = datagen.small(4, nq=8, n_seq=8, l_max=16384)
    _misa_case(dsa, wl, h=8, k=256, kprime=1024)


def test_misa_partial_blocks_and_internal_pooling(dsa):
    """Queries on one shared cache at positions that end inside a block: the
    partial last block is pooled over its valid tokens only; the call pools the
    cache itself when no pooled keys are given."""
    wl = datagen.small(4, nq=6, n_seq=1, l_max=9000, layout="tail", plant="points", n_plant=60)
    pos = [0, 63, 64, 100, 4097, 8999]
    for pooled in (True, False):
        _misa_case(dsa, wl, h=8, k=128, kprime=512, pos=pos, pooled=pooled)
        _misa_case(dsa, wl, h=3, k=50, kprime=0, pos=pos, pooled=pooled)


def test_misa_many_queries_one_router_slice(dsa):
    """More queries than the router's workgroup target: every query's blocks fit
    one router slice (the plan stops widening slices there)."""
    wl = datagen.small(4, nq=600, n_seq=600, l_max=2048)
    rows = list(range(0, 600, 37)) + [599]
    _misa_case(dsa, wl, h=12, k=128, kprime=256, rows=rows)


def _misa_prefill_wl(nq, L, **kw):
    # MISA's values on the prefill layout: row t at position t of one sequence
    return datagen.small(4, nq=nq, n_seq=1, l_max=L, layout="prefill", plant="points",
                         n_plant=max(8, nq // 8), **kw)


def test_misa_prefill_rows(dsa):
    """MISA on the prefill shape (many rows of one sequence, h <= 8): the router,
    the head selection, the packed routed scoring and the row select.  512 rows
    with a 64-key block: rows end inside a block (partial last blocks), rows
    0..63 are shorter than k."""
    wl = _misa_prefill_wl(512, 512)
    _misa_case(dsa, wl, h=8, k=64, kprime=0)


def test_misa_prefill_larger_and_fewer_heads(dsa):
    wl = _misa_prefill_wl(2048, 2048)
    rows = list(range(0, 2048, 41)) + [2047]
    _misa_case(dsa, wl, h=8, k=300, kprime=0, seed=1, rows=rows)
    _misa_case(dsa, wl, h=3, k=300, kprime=0, seed=2, rows=rows, pooled=False)
    _misa_case(dsa, wl, h=1, k=100, kprime=0, seed=3, rows=rows)


def test_misa_prefill_heads_and_dims(dsa):
    for H, d, h in ((32, 128, 8), (64, 64, 5), (16, 128, 7)):
        wl = _misa_prefill_wl(256, 700, n_heads=H, head_dim=d)
        _misa_case(dsa, wl, h=h, k=100, kprime=0, seed=4)


def test_misa_prefill_arbitrary_positions_and_invalid_rows(dsa):
    """Positions in any order and rows that are not valid for a one-sequence call."""
    wl = _misa_prefill_wl(100, 3000)
    rng = np.random.default_rng(5)
    pos = rng.integers(0, 3000, size=100)
    pos[5], pos[6], pos[7], pos[8] = -1, 3000, 2999, 0
    inp = datagen.make(wl, 6)
    inp["q_pos"] = pos.astype(np.int32)
    dev = upload(inp, wl)
    res = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], None, block=64,
                                    n_active_heads=8, top_k=256)
    gi = res["idx"].cpu().numpy()
    heads = res["heads"].cpu().numpy()
    for t in (5, 6):
        assert np.all(gi[t] == -1) and np.all(heads[t] == -1), f"invalid row {t}"
    valid = [t for t in range(100) if t not in (5, 6)]
    _misa_case(dsa, wl, h=8, k=256, kprime=0, seed=6, pos=pos, rows=valid)


def test_misa_shared_cache_decode_queries(dsa):
    """MISA for 64 decode queries sharing one 131072-key cache (its last 64
    positions, most ending inside a 64-key block): the prefill-shaped router
    and the routed scorer with its keys split over workgroups (rows longer than
    65535 keys); every query's heads, then its selection given those heads."""
    wl = datagen.small(4, nq=64, n_seq=1, l_max=131072, layout="tail", plant="points",
                       n_plant=64)
    _misa_case(dsa, wl, h=8, k=2048, kprime=0, seed=12)


def test_misa_all_heads_equals_dense(dsa):
    """h = H_I routes every head: the selection must be the dense indexer's."""
    wl = datagen.small(4, nq=4, n_seq=4, l_max=8192)
    inp = datagen.make(wl, 2)
    dev = upload(inp, wl)
    res = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    block=64, n_active_heads=64, top_k=300)
    gi, gv = res["idx"].cpu().numpy(), res["score"].cpu().numpy()
    errs = []
    for t in range(4):
        q_t, w_t, K, p = _rows(inp, wl, t)
        d = O.dense_row(q_t, w_t, K, p, 300)
        errs += _check(gi[t], gv[t], d["cand"], d["s"], d["A"], 300, q_t, w_t, K, f"q{t}")
    assert not errs, "\n".join(errs[:8])


def test_misa_dagger_full_candidate_set_equals_dense(dsa):
    """k' >= prefix length keeps every token, so the rescored top-k is dense."""
    wl = datagen.small(4, nq=4, n_seq=4, l_max=3000)
    inp = datagen.make(wl, 3)
    dev = upload(inp, wl)
    res = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    block=64, n_active_heads=8, top_k=200, k_prime=4096)
    gi, gv = res["idx"].cpu().numpy(), res["score"].cpu().numpy()
    errs = []
    for t in range(4):
        q_t, w_t, K, p = _rows(inp, wl, t)
        d = O.dense_row(q_t, w_t, K, p, 200)
        errs += _check(gi[t], gv[t], d["cand"], d["s"], d["A"], 200, q_t, w_t, K, f"q{t}")
    assert not errs, "\n".join(errs[:8])


def _hisa_case(dsa, wl, m, k, seed=0, pos=None, pooled=True, rows=None):
    inp = datagen.make(wl, seed)
    if pos is not None:
        inp["q_pos"] = np.asarray(pos, dtype=np.int32)
    say(f"[hisa] nq={wl.nq} L={wl.l_max} H={wl.n_heads} B={wl.block} m={m} k={k} pooled={pooled}")
    dev = upload(inp, wl)
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block) if pooled else None
    res = dsa.hisa_block_filter_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                     block=wl.block, m_blocks=m, top_k=k, k_pooled=kp)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in res.items()}
    errs = [] if not out["status"].any() else [f"status {out['status'].tolist()[:16]}"]
    for t in (range(wl.nq) if rows is None else rows):
        q_t, w_t, K, p = _rows(inp, wl, t)
        pooled_ref = O.misa_pooled_for_query(K, wl.block, p)
        bs, bA = O.hisa_block_scores(q_t, w_t, pooled_ref)
        Fb = O.dot_magnitude(q_t, w_t, pooled_ref)
        errs += check_selection(out["blocks"][t], out["block_score"][t],
                                np.arange(pooled_ref.shape[0]), bs, bA, m, Fb, what=f"blocks q{t}")
        r = O.hisa_row(q_t, w_t, K, p, wl.block, m, k, blocks=out["blocks"][t])
        errs += _check(out["idx"][t], out["score"][t], r["cand"], r["s"], r["A"], k,
                       q_t, w_t, K, f"hisa q{t}")
    assert not errs, "\n".join(errs[:12])
    return inp, out


def test_hisa_reduced(dsa):
    wl = datagen.small(5, nq=8, n_seq=8, l_max=65536, n_plant=48)
    _hisa_case(dsa, wl, m=16, k=512)


def test_hisa_partial_blocks_and_internal_pooling(dsa):
    wl = datagen.small(5, nq=6, n_seq=1, l_max=9000, layout="tail", plant="points", n_plant=60)
    pos = [0, 127, 128, 300, 4097, 8999]
    for pooled in (True, False):
        _hisa_case(dsa, wl, m=8, k=200, pos=pos, pooled=pooled)


def test_hisa_prefill_rows(dsa):
    """HISA on the prefill layout: many rows of one sequence at positions
    0..nq-1, so early rows keep every block (fewer than m), rows end inside a
    block (partial last block pooled over the row's tokens), and rows with
    fewer than k candidate tokens are padded."""
    wl = datagen.small(5, nq=1024, n_seq=1, l_max=1024, layout="prefill", plant="points",
                       n_plant=128, block=64)
    rows = list(range(0, 1024, 37)) + [63, 64, 65, 1023]
    _hisa_case(dsa, wl, m=6, k=200, rows=rows)
    _hisa_case(dsa, wl, m=3, k=64, seed=1, rows=rows, pooled=False)


def test_hisa_heads_dims_and_the_multi_launch_path(dsa):
    """The fused kernel's other scorers (16 heads: one 16-row tile; 64 heads:
    two 32-row tiles; d = 64), and m * B above 8192 (the multi-launch path)."""
    for H, d in ((16, 128), (64, 128), (48, 64)):
        wl = datagen.small(5, nq=4, n_seq=4, l_max=30000, n_plant=48, n_heads=H, head_dim=d)
        _hisa_case(dsa, wl, m=24, k=400, seed=H + d)
    wl = datagen.small(5, nq=3, n_seq=3, l_max=40000, n_plant=60, block=64)
    _hisa_case(dsa, wl, m=200, k=1000, seed=7)


def test_hisa_wait_timeout_is_reported(dsa):
    """The token pass's bounded wait, forced from the host to give up at its
    first unsuccessful check (wait limit 0): every kernel still ends normally;
    a query whose wait gave up reports status 1 and a row of padding only
    (never a partial selection) while its kept blocks are still exact; every
    other query's row is the exact selection.  The same workspace then serves
    a call with the default limit, which completes every query."""
    wl = datagen.small(5, nq=8, n_seq=8, l_max=65536, n_plant=48)
    m, k = 16, 512
    inp = datagen.make(wl, 0)
    dev = upload(inp, wl)
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block)
    nb = dsa.hisa_block_filter_topk_workspace_size(wl.nq, wl.n_heads, wl.head_dim, wl.n_seq,
                                                   wl.l_max, wl.block, m, k, 1)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:][:nb]
    args = (dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"])
    say("[hisa] wait limit 0")
    dsa.hisa_wait_limit(0)
    try:
        res0 = dsa.hisa_block_filter_topk(*args, block=wl.block, m_blocks=m, top_k=k, k_pooled=kp,
                                          workspace=ws)
        mh0 = dsa.misa_hisa_topk(*args, block=wl.block, n_active_heads=8, m_blocks=m, top_k=k,
                                 k_pooled=kp)
        torch.cuda.synchronize()
    finally:
        dsa.hisa_wait_limit(-1)
    res1 = dsa.hisa_block_filter_topk(*args, block=wl.block, m_blocks=m, top_k=k, k_pooled=kp,
                                      workspace=ws)
    torch.cuda.synchronize()
    o0 = {x: v.cpu().numpy() for x, v in res0.items()}
    o1 = {x: v.cpu().numpy() for x, v in res1.items()}
    mh = {x: v.cpu().numpy() for x, v in mh0.items()}
    say(f"[hisa] timed-out queries: hisa {o0['status'].tolist()} misa-hisa {mh['status'].tolist()}")
    assert set(o0["status"].tolist()) <= {0, 1} and set(mh["status"].tolist()) <= {0, 1}
    # 64 token-pass workgroups per query, all but the selecting one check for
    # the kept blocks before the selection can have been published
    assert o0["status"].sum() > 0 and mh["status"].sum() > 0
    assert not o1["status"].any()
    errs = []
    for t in range(wl.nq):
        q_t, w_t, K, p = _rows(inp, wl, t)
        pooled_ref = O.misa_pooled_for_query(K, wl.block, p)
        bs, bA = O.hisa_block_scores(q_t, w_t, pooled_ref)
        Fb = O.dot_magnitude(q_t, w_t, pooled_ref)
        for o, tag in ((o0, "limited"), (o1, "default")):
            errs += check_selection(o["blocks"][t], o["block_score"][t],
                                    np.arange(pooled_ref.shape[0]), bs, bA, m, Fb,
                                    what=f"{tag} blocks q{t}")
            if o["status"][t]:
                if (o["idx"][t] != -1).any() or not np.isneginf(o["score"][t]).all():
                    errs.append(f"{tag} q{t}: timed out but the row is not all padding")
                continue
            r = O.hisa_row(q_t, w_t, K, p, wl.block, m, k, blocks=o["blocks"][t])
            errs += _check(o["idx"][t], o["score"][t], r["cand"], r["s"], r["A"], k,
                           q_t, w_t, K, f"{tag} hisa q{t}")
        if mh["status"][t] and ((mh["idx"][t] != -1).any() or not np.isneginf(mh["score"][t]).all()):
            errs.append(f"misa-hisa q{t}: timed out but the row is not all padding")
    assert not errs, "\n".join(errs[:12])


def _misa_hisa_case(dsa, wl, h, m, k, seed=0, pos=None, pooled=True, rows=None):
    inp = datagen.make(wl, seed)
    if pos is not None:
        inp["q_pos"] = np.asarray(pos, dtype=np.int32)
    say(f"[misa-hisa] nq={wl.nq} L={wl.l_max} H={wl.n_heads} B={wl.block} h={h} m={m} k={k} "
        f"pooled={pooled}")
    dev = upload(inp, wl)
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block) if pooled else None
    res = dsa.misa_hisa_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                             block=wl.block, n_active_heads=h, m_blocks=m, top_k=k, k_pooled=kp,
                             with_importance=True)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in res.items()}
    errs = []
    for t in (range(wl.nq) if rows is None else rows):
        q_t, w_t, K, p = _rows(inp, wl, t)
        pooled_ref = O.misa_pooled_for_query(K, wl.block, p)
        I = O.misa_importance(q_t, w_t, pooled_ref)
        Fi = np.abs(w_t) * (np.abs(q_t) @ np.abs(pooled_ref).T).sum(axis=1)
        gi = out["importance"][t].astype(np.float64)
        bad = ~scores_ok(gi, I, I, Fi)
        if bad.any():
            errs.append(f"importance q{t}: heads {np.nonzero(bad)[0][:4]}")
        errs += check_selection(out["heads"][t], None, np.arange(wl.n_heads), I, I, h, Fi,
                                what=f"heads q{t}")
        heads = out["heads"][t].astype(np.int64)
        # blocks, given the GPU's heads
        bs, bA = O.hisa_block_scores(q_t[heads], w_t[heads], pooled_ref)
        Fb = O.dot_magnitude(q_t[heads], w_t[heads], pooled_ref)
        errs += check_selection(out["blocks"][t], out["block_score"][t],
                                np.arange(pooled_ref.shape[0]), bs, bA, m, Fb,
                                what=f"blocks q{t}")
        # tokens, given the GPU's heads and blocks
        r = O.misa_hisa_row(q_t, w_t, K, p, wl.block, h, m, k, heads=heads,
                            blocks=out["blocks"][t])
        errs += _check(out["idx"][t], out["score"][t], r["cand"], r["s"], r["A"], k,
                       q_t, w_t, K, f"misa-hisa q{t}", heads)
    assert not errs, "\n".join(errs[:12])


def test_misa_hisa_reduced(dsa):
    wl = datagen.small(5, nq=8, n_seq=8, l_max=65536, n_plant=48)
    _misa_hisa_case(dsa, wl, h=8, m=16, k=512)


def test_misa_hisa_partial_blocks_internal_pooling_and_prefill_rows(dsa):
    wl = datagen.small(5, nq=6, n_seq=1, l_max=9000, layout="tail", plant="points", n_plant=60)
    _misa_hisa_case(dsa, wl, h=4, m=8, k=200, pos=[0, 127, 128, 300, 4097, 8999], pooled=False)
    wl = datagen.small(5, nq=1024, n_seq=1, l_max=1024, layout="prefill", plant="points",
                       n_plant=128, block=64)
    _misa_hisa_case(dsa, wl, h=3, m=6, k=200, rows=list(range(0, 1024, 41)) + [63, 64, 1023])


def test_misa_hisa_wider_routes_and_head_dims(dsa):
    """Routed head counts that select the wider scorers (h = 24 of 32: one
    32-row tile; h = 40 of 64: two tiles) and d = 64."""
    wl = datagen.small(5, nq=4, n_seq=4, l_max=32768, n_plant=48)
    _misa_hisa_case(dsa, wl, h=24, m=16, k=300, seed=1)
    wl = datagen.small(5, nq=4, n_seq=4, l_max=32768, n_plant=48, n_heads=64)
    _misa_hisa_case(dsa, wl, h=40, m=16, k=300, seed=2)
    wl = datagen.small(5, nq=4, n_seq=4, l_max=20000, n_plant=48, head_dim=64)
    _misa_hisa_case(dsa, wl, h=5, m=32, k=500, seed=3)


def test_misa_hisa_argument_errors(dsa):
    """Calls the library rejects before any launch."""
    wl = datagen.small(5, nq=2, n_seq=2, l_max=4096)
    dev = upload(datagen.make(wl, 0), wl)
    args = (dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"])
    for h, m in ((0, 8), (wl.n_heads + 1, 8), (4, 0), (4, 1025), (4, 100)):
        # h out of range, no blocks, more blocks than supported, m * B > 8192
        with pytest.raises(dsa.DsaError):
            dsa.misa_hisa_topk(*args, block=128, n_active_heads=h, m_blocks=m, top_k=64)


def test_hisa_exact_ties_take_lowest_ids(dsa):
    """Zero queries make every block and token score exactly 0.0, so both
    selections are decided by the tie-break alone (lower index first): the
    kept blocks are 0..m-1 and the tokens the k lowest of theirs.  With 4096
    blocks per query (every block a candidate) and a tie bin holding every
    token item, this runs the selection paths for candidate lists and tie
    bins that do not fit in LDS; one query ends inside a block."""
    n_seq, L, H, D, B, m, k = 4, 262144, 32, 128, 64, 64, 1000
    pos = np.array([L - 1, L - 18, 100000, 5000], dtype=np.int32)
    say(f"[hisa ties] nq={n_seq} L={L} H={H} B={B} m={m} k={k}")
    g = torch.Generator(device="cuda").manual_seed(3)
    q = torch.zeros((n_seq, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((n_seq, H), device="cuda", generator=g)
    keys = torch.randn((n_seq, L, D), device="cuda", generator=g).to(torch.bfloat16)
    res = dsa.hisa_block_filter_topk(q, w, keys, torch.from_numpy(pos).cuda(),
                                     torch.arange(n_seq, dtype=torch.int32, device="cuda"),
                                     block=B, m_blocks=m, top_k=k)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in res.items()}
    errs = []
    for t in range(n_seq):
        M = (int(pos[t]) + B) // B
        mb = min(m, M)
        if sorted(out["blocks"][t][:mb].tolist()) != list(range(mb)):
            errs.append(f"q{t}: blocks {sorted(out['blocks'][t][:mb].tolist())[:8]}...")
        if np.any(out["block_score"][t][:mb] != 0.0):
            errs.append(f"q{t}: block scores not all zero")
        toks = np.arange(mb * B)
        toks = toks[toks <= pos[t]]
        kt = min(k, toks.size)
        if sorted(out["idx"][t][:kt].tolist()) != toks[:kt].tolist():
            errs.append(f"q{t}: tokens {sorted(out['idx'][t][:kt].tolist())[:8]}...")
        if np.any(out["score"][t][:kt] != 0.0) or np.any(out["idx"][t][kt:] != -1):
            errs.append(f"q{t}: token scores not zero or padding wrong")
    assert not errs, "\n".join(errs)


def test_hisa_all_blocks_equals_dense_and_iou(dsa):
    """m >= M keeps every block, so HISA equals dense; with m < M the IoU kernel
    agrees with the oracle's IoU of the same two selections."""
    wl = datagen.small(5, nq=4, n_seq=4, l_max=16384, n_plant=24)
    inp = datagen.make(wl, 4)
    dev = upload(inp, wl)
    M = 16384 // wl.block
    res = dsa.hisa_block_filter_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                     block=wl.block, m_blocks=M, top_k=256)
    dn, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"], top_k=256)
    gi, gv = res["idx"].cpu().numpy(), res["score"].cpu().numpy()
    errs = []
    for t in range(4):
        q_t, w_t, K, p = _rows(inp, wl, t)
        d = O.dense_row(q_t, w_t, K, p, 256)
        errs += _check(gi[t], gv[t], d["cand"], d["s"], d["A"], 256, q_t, w_t, K, f"q{t}")
    assert not errs, "\n".join(errs[:8])
    small = dsa.hisa_block_filter_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                       block=wl.block, m_blocks=8, top_k=256)
    iou = dsa.indexer_selection_iou(small["idx"], dn).cpu().numpy()
    ref = O.iou_rows(small["idx"].cpu().numpy(), dn.cpu().numpy())
    np.testing.assert_allclose(iou, ref, rtol=1e-6)


def _by_groups(ids, labels, gscore, kk, what):
    """The kk items of largest group score, ties to the lower id; identical key
    rows give bit-identical scores on both sides, so this set is exact as long
    as the groups around the k-th place are farther apart than the tolerance
    (asserted, so that an input too close to call fails loudly)."""
    order = sorted(range(len(ids)), key=lambda i: (-gscore[labels[i]], ids[i]))
    kk = min(kk, len(ids))
    if kk < len(ids):
        g = labels[order[kk - 1]]
        vals = sorted({float(gscore[x]) for x in set(labels.tolist())}, reverse=True)
        j = vals.index(float(gscore[g]))
        tol = 2e-3 * abs(vals[j]) + 1e-6
        near = [abs(vals[j] - vals[i]) for i in (j - 1, j + 1) if 0 <= i < len(vals)]
        assert min(near, default=np.inf) > 4 * tol, \
            f"{what}: groups around the k-th place too close to call"
    return sorted(int(ids[i]) for i in order[:kk])


@pytest.mark.parametrize("per_block", [False, True])
def test_hisa_few_distinct_key_rows_resolve_ties_by_index(dsa, per_block):
    """Keys drawn from a small palette of distinct rows (per token: 24 rows; per
    block: 8 rows, every token of a block the same row).  Identical rows score
    identically, so the k-th token score's bin holds one tied row's items
    (about 170 of 4096, or 512) and, per block, the m-th block score's bin
    about 128 tied blocks: both selections resolve large tie bins, which must
    keep every item of the higher-scoring rows and, of the tied row, the lowest
    indices.  Scores are checked against the oracle under the usual rule."""
    n_seq, L, H, D, B, m, k = 4, 65536, 32, 128, 64, 64, 1000
    P = 8 if per_block else 24
    rng = np.random.default_rng(21 if per_block else 22)
    pos = np.array([L - 1, L - 30, 40000, 9000], dtype=np.int32)
    say(f"[hisa palette] per_block={per_block} P={P} nq={n_seq} L={L} B={B} m={m} k={k}")
    pal = torch.from_numpy(rng.standard_normal((P, D)).astype(np.float32)).to(torch.bfloat16)
    lab = (np.repeat(rng.integers(0, P, size=(n_seq, L // B)), B, axis=1) if per_block
           else rng.integers(0, P, size=(n_seq, L)))
    q = torch.from_numpy(rng.standard_normal((n_seq, H, D)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((n_seq, H)).astype(np.float32))
    keys = pal[torch.from_numpy(lab)]                                   # [n_seq, L, D]
    res = dsa.hisa_block_filter_topk(q.cuda(), w.cuda(), keys.cuda(), torch.from_numpy(pos).cuda(),
                                     torch.arange(n_seq, dtype=torch.int32, device="cuda"),
                                     block=B, m_blocks=m, top_k=k)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in res.items()}
    errs = [] if not out["status"].any() else [f"status {out['status'].tolist()}"]
    bits = lambda x: x.view(torch.int16).numpy().view(np.uint16)
    pal64 = O.to_f64(bits(pal), datagen.BF16)
    K_all = O.to_f64(bits(keys), datagen.BF16)
    for t in range(n_seq):
        q_t = O.to_f64(bits(q[t]), datagen.BF16)
        w_t = w[t].numpy().astype(np.float64)
        p = int(pos[t])
        gs, _ = O.hisa_block_scores(q_t, w_t, pal64)                      # score of each row
        M = (p + B) // B
        if per_block:                                                  # blocks: exact set
            want = _by_groups(np.arange(M), lab[t, ::B][:M], gs, m, f"blocks q{t}")
            got = sorted(out["blocks"][t][:min(m, M)].tolist())
            if got != want:
                errs.append(f"q{t}: blocks differ from the tie rule ({len(set(got) ^ set(want))})")
        K = K_all[t]
        pooled_ref = O.misa_pooled_for_query(K, B, p)
        bs, bA = O.hisa_block_scores(q_t, w_t, pooled_ref)
        errs += check_selection(out["blocks"][t], out["block_score"][t], np.arange(M), bs, bA, m,
                                O.dot_magnitude(q_t, w_t, pooled_ref), what=f"blocks q{t}")
        r = O.hisa_row(q_t, w_t, K, p, B, m, k, blocks=out["blocks"][t])
        errs += _check(out["idx"][t], out["score"][t], r["cand"], r["s"], r["A"], k, q_t, w_t, K,
                       f"hisa q{t}")
        cand = r["cand"]
        want = _by_groups(cand, lab[t][cand], gs, k, f"tokens q{t}")
        got = sorted(out["idx"][t][:min(k, cand.size)].tolist())
        if got != want:
            errs.append(f"q{t}: tokens differ from the tie rule ({len(set(got) ^ set(want))})")
    assert not errs, "\n".join(errs[:12])
