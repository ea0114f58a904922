"""GPU parity at the full workload sizes, in the launch configuration bench.py
times; the oracle checks sampled queries one by one (keys of the sampled
queries' sequences are regenerated on the host from the same seeds)."""
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import datagen
from oracle import indexer as O
from oracle.check import check_selection, scores_ok

from _helpers import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_indexer_amd as m
    m.lib()
    return m


def _device_inputs(wl, seed=0, per_seq=None):
    """q, w, positions on the device; K generated per sequence straight into a
    device tensor (host memory stays at one sequence per worker).  per_seq(s,
    keys of s), if given, runs in the worker on each sequence's host keys; its
    results come back as a list (oracle work that needs every sequence's keys)."""
    q, w = datagen.queries(wl, seed)
    q_seq, q_pos = datagen.positions(wl)
    kdev = torch.empty((wl.n_seq, wl.l_max, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    extra = [None] * wl.n_seq

    def gen(s):
        ks = datagen.keys(wl, s, q, w, seed)
        if per_seq is not None:
            extra[s] = per_seq(s, ks, q, w)
        return ks

    with ThreadPoolExecutor(max_workers=16) as ex:
        for s, ks in enumerate(ex.map(gen, range(wl.n_seq))):
            kdev[s].copy_(to_device(ks, wl.dtype))
    dev = {"q": to_device(q, wl.dtype), "w": torch.from_numpy(w).cuda(), "k": kdev,
           "q_seq": torch.from_numpy(q_seq).cuda(), "q_pos": torch.from_numpy(q_pos).cuda()}
    host = {"q": q, "w": w, "q_seq": q_seq, "q_pos": q_pos}
    if per_seq is not None:
        host["per_seq"] = extra
    return dev, host


def _dense_topk_of_own_query(wl):
    """per_seq hook for the decode layout (query t on sequence t at l_max - 1):
    the oracle's dense top-k of that query."""
    def f(s, ks, q, w):
        t = s
        r = O.dense_row(O.to_f64(q[t], wl.dtype), w[t].astype(np.float64), O.to_f64(ks, wl.dtype),
                        wl.l_max - 1, wl.top_k)
        return r["idx"].astype(np.int32)
    return f


def _iou_report(dsa, name, gpu_idx, ref_idx):
    """IoU of a variant's selection against a dense selection, per query: the
    GPU kernel's value must equal the oracle's; prints mean and min."""
    g = dsa.indexer_selection_iou(torch.from_numpy(np.ascontiguousarray(gpu_idx, np.int32)).cuda(),
                                  torch.from_numpy(np.ascontiguousarray(ref_idx, np.int32)).cuda())
    g = g.cpu().numpy().astype(np.float64)
    o = O.iou_rows(gpu_idx, ref_idx)
    np.testing.assert_allclose(g, o, rtol=1e-6, atol=1e-7)
    say(f"[iou] {name}: mean {o.mean():.4f} min {o.min():.4f} max {o.max():.4f} over {o.size} queries")
    return o


def _host_row(wl, hostin, t, seed=0):
    s = int(hostin["q_seq"][t])
    K = O.to_f64(datagen.keys(wl, s, hostin["q"], hostin["w"], seed), wl.dtype)
    return O.to_f64(hostin["q"][t], wl.dtype), hostin["w"][t].astype(np.float64), K, int(hostin["q_pos"][t])


def _rows_parallel(fn, rows, workers=16):
    """fn(t) -> list of failure strings, over the rows in a thread pool (the
    oracle's NumPy work releases the interpreter lock); failures in row order."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return [e for errs in ex.map(fn, rows) for e in errs]


# what only the float32 rounding fallback of the matching rule admitted, per test
_FALLBACK = {}
_FALLBACK_LOCK = threading.Lock()


@pytest.fixture(autouse=True)
def _fallback_report():
    _FALLBACK.clear()
    yield
    say(f"[checker] admitted only by the rounding bound: {dict(_FALLBACK)}")


def _check(gi, gv, r, k, q_t, w_t, K, what, heads=None):
    qq, ww = (q_t, w_t) if heads is None else (q_t[heads], w_t[heads])
    F = O.dot_magnitude(qq, ww, K[r["cand"]])
    st = {}
    errs = check_selection(gi, gv, r["cand"], r["s"], r["A"], k, F, what=what, stats=st)
    with _FALLBACK_LOCK:               # (rows are checked on several threads)
        for key, v in st.items():
            _FALLBACK[key] = _FALLBACK.get(key, 0) + v
    return errs


def test_dense_decode_full(dsa):
    """64 queries x 131072 keys, 64 heads, d 128, bf16, k 2048: every query."""
    wl = datagen.WORKLOADS[2]
    say("[full] dense decode 64 x 131072")
    dev, h = _device_inputs(wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=wl.top_k)
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    errs = []
    for t in range(wl.nq):
        q_t, w_t, K, p = _host_row(wl, h, t)
        r = O.dense_row(q_t, w_t, K, p, wl.top_k)
        errs += _check(gi[t], gv[t], r, wl.top_k, q_t, w_t, K, f"q{t}")
    assert not errs, "\n".join(errs[:10])


def test_misa_full(dsa):
    """64 x 131072, B 64, h 8 of 64 heads, k 2048 (MISA) and k' 8192 (dagger);
    every query, each stage on the GPU's own upstream choice; the dense call on
    the same inputs and the IoU of both variants against it."""
    wl = datagen.WORKLOADS[4]
    say("[full] MISA 64 x 131072")
    dev, h = _device_inputs(wl)
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block)
    m = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                  block=wl.block, n_active_heads=wl.n_active_heads,
                                  top_k=wl.top_k, k_pooled=kp)
    md = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                   block=wl.block, n_active_heads=wl.n_active_heads,
                                   top_k=wl.top_k, k_prime=wl.k_prime, k_pooled=kp, with_cand=True)
    dn, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                   top_k=wl.top_k, with_scores=False)
    mi, mv, heads = (m[x].cpu().numpy() for x in ("idx", "score", "heads"))
    di, dv, cand, dheads = (md[x].cpu().numpy() for x in ("idx", "score", "cand", "heads"))
    dni = dn.cpu().numpy()
    assert np.array_equal(heads, dheads)
    # selection agreement with the dense indexer on the same inputs (MISA
    # summary, "results": the pages report MISA dagger above 92 % per layer)
    _iou_report(dsa, "MISA h=8 vs dense (64 x 131072)", mi, dni)
    _iou_report(dsa, "MISA dagger k'=8192 vs dense (64 x 131072)", di, dni)

    def row(t):
        errs = []
        q_t, w_t, K, p = _host_row(wl, h, t)
        pooled = O.misa_pooled_for_query(K, wl.block, p)
        I = O.misa_importance(q_t, w_t, pooled)
        errs += check_selection(heads[t], None, np.arange(wl.n_heads), I, I, wl.n_active_heads,
                                what=f"heads q{t}")
        hs = heads[t].astype(np.int64)
        r = O.misa_row(q_t, w_t, K, p, wl.block, wl.n_active_heads, wl.k_prime, heads=hs)
        errs += _check(cand[t], None, r, wl.k_prime, q_t, w_t, K, f"coarse q{t}", hs)
        rk = dict(r)
        errs += _check(mi[t], mv[t], rk, wl.top_k, q_t, w_t, K, f"misa q{t}", hs)
        f = O.rescore_row(q_t, w_t, K, cand[t], wl.top_k)
        errs += _check(di[t], dv[t], f, wl.top_k, q_t, w_t, K, f"dagger q{t}")
        d = O.dense_row(q_t, w_t, K, p, wl.top_k)
        errs += _check(dni[t], None, d, wl.top_k, q_t, w_t, K, f"dense q{t}")
        return errs

    errs = _rows_parallel(row, range(wl.nq))      # every query
    assert not errs, "\n".join(errs[:10])


@pytest.mark.skip(reason="one run of this test faulted the GPU (illegal address) right after a "
                         "workspace-plan change that was taken out uncommitted; the host-side bounds "
                         "audit (tests/test_audit_cpu.py) finds every access of its three calls inside "
                         "its buffers, but no cause of the fault is shown, so the case stays off the "
                         "GPU; the IoU it measured is taken against the oracle's dense selection in "
                         "test_hisa_and_misa_hisa_full_all_rows")
def test_hisa_full_with_iou(dsa):
    """32 queries x 1048576 keys, 32 heads, B 128, m 64, k 2048; IoU against the
    dense 32-head indexer on the same inputs."""
    wl = datagen.WORKLOADS[5]
    say("[full] HISA 32 x 1048576")
    dev, h = _device_inputs(wl)
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block)
    r = dsa.hisa_block_filter_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                   block=wl.block, m_blocks=wl.m_blocks, top_k=wl.top_k, k_pooled=kp)
    dn, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                   top_k=wl.top_k)
    iou = dsa.indexer_selection_iou(r["idx"], dn).cpu().numpy()
    hi, hv, blocks, bsc = (r[x].cpu().numpy() for x in ("idx", "score", "blocks", "block_score"))
    dni = dn.cpu().numpy()
    np.testing.assert_allclose(iou, O.iou_rows(hi, dni), rtol=1e-6)
    say(f"[full] HISA IoU vs dense: mean {iou.mean():.4f} min {iou.min():.4f}")
    errs = []
    for t in (0, 13, 31):
        q_t, w_t, K, p = _host_row(wl, h, t)
        pooled = O.misa_pooled_for_query(K, wl.block, p)
        bs, bA = O.hisa_block_scores(q_t, w_t, pooled)
        errs += check_selection(blocks[t], bsc[t], np.arange(pooled.shape[0]), bs, bA, wl.m_blocks,
                                O.dot_magnitude(q_t, w_t, pooled), what=f"blocks q{t}")
        rr = O.hisa_row(q_t, w_t, K, p, wl.block, wl.m_blocks, wl.top_k, blocks=blocks[t])
        errs += _check(hi[t], hv[t], rr, wl.top_k, q_t, w_t, K, f"hisa q{t}")
        d = O.dense_row(q_t, w_t, K, p, wl.top_k)
        errs += _check(dni[t], None, d, wl.top_k, q_t, w_t, K, f"dense q{t}")
    assert not errs, "\n".join(errs[:10])


def test_hisa_and_misa_hisa_full_all_rows(dsa):
    """32 queries x 1048576 keys, 32 heads, B 128, m 64, k 2048, as timed: the
    pooling, HISA over all heads and MISA∘HISA with h = 8 (the three calls of
    the hisa and misa_hisa workloads).  Every query against the oracle, each
    stage conditional on the GPU's own upstream choice; the IoU of both
    variants against the oracle's dense top-k of every query."""
    wl = datagen.WORKLOADS[5]
    h_act = 8
    say("[full] HISA and MISA∘HISA 32 x 1048576")
    dev, h = _device_inputs(wl, per_seq=_dense_topk_of_own_query(wl))
    args = (dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"])
    kp = dsa.indexer_mean_pool_keys(dev["k"], wl.block)
    r = dsa.hisa_block_filter_topk(*args, block=wl.block, m_blocks=wl.m_blocks, top_k=wl.top_k,
                                   k_pooled=kp)
    mh = dsa.misa_hisa_topk(*args, block=wl.block, n_active_heads=h_act, m_blocks=wl.m_blocks,
                            top_k=wl.top_k, k_pooled=kp, with_importance=True)
    torch.cuda.synchronize()
    hi, hv, blocks, bsc = (r[x].cpu().numpy() for x in ("idx", "score", "blocks", "block_score"))
    out = {x: v.cpu().numpy() for x, v in mh.items()}
    assert not r["status"].cpu().numpy().any() and not out["status"].any()
    # selection agreement with the dense 32-head indexer on every query, the
    # dense top-k taken by the oracle (HISA review, section 3: above 99 % on
    # the pages' models)
    dense_ref = np.stack(h["per_seq"])
    _iou_report(dsa, "HISA m=64 vs dense (32 x 1048576)", hi, dense_ref)
    _iou_report(dsa, "MISA∘HISA h=8 m=64 vs dense (32 x 1048576)", out["idx"], dense_ref)

    def row(t):
        errs = []
        q_t, w_t, K, p = _host_row(wl, h, t)
        pooled = O.misa_pooled_for_query(K, wl.block, p)
        # HISA: blocks, then tokens inside the GPU's blocks
        bs, bA = O.hisa_block_scores(q_t, w_t, pooled)
        errs += check_selection(blocks[t], bsc[t], np.arange(pooled.shape[0]), bs, bA, wl.m_blocks,
                                O.dot_magnitude(q_t, w_t, pooled), what=f"hisa blocks q{t}")
        rr = O.hisa_row(q_t, w_t, K, p, wl.block, wl.m_blocks, wl.top_k, blocks=blocks[t])
        errs += _check(hi[t], hv[t], rr, wl.top_k, q_t, w_t, K, f"hisa q{t}")
        # MISA∘HISA: importance and heads, blocks with the GPU's heads, tokens
        I = O.misa_importance(q_t, w_t, pooled)
        Fi = np.abs(w_t) * (np.abs(q_t) @ np.abs(pooled).T).sum(axis=1)
        gi = out["importance"][t].astype(np.float64)
        if not scores_ok(gi, I, I, Fi).all():
            errs.append(f"misa-hisa importance q{t}")
        errs += check_selection(out["heads"][t], None, np.arange(wl.n_heads), I, I, h_act, Fi,
                                what=f"misa-hisa heads q{t}")
        hs = out["heads"][t].astype(np.int64)
        bs2, bA2 = O.hisa_block_scores(q_t[hs], w_t[hs], pooled)
        errs += check_selection(out["blocks"][t], out["block_score"][t], np.arange(pooled.shape[0]),
                                bs2, bA2, wl.m_blocks, O.dot_magnitude(q_t[hs], w_t[hs], pooled),
                                what=f"misa-hisa blocks q{t}")
        r2 = O.misa_hisa_row(q_t, w_t, K, p, wl.block, h_act, wl.m_blocks, wl.top_k, heads=hs,
                             blocks=out["blocks"][t])
        errs += _check(out["idx"][t], out["score"][t], r2, wl.top_k, q_t, w_t, K,
                       f"misa-hisa q{t}", hs)
        return errs

    errs = _rows_parallel(row, range(wl.nq))      # every query
    assert not errs, "\n".join(errs[:10])


def _prefill_rows(edges, seed, n=248, L=32768):
    """The edge rows plus n more drawn (seeded, without repeats) from the whole
    triangle, in order."""
    extra = np.random.default_rng(seed).choice(L, size=n, replace=False)
    return sorted(set(edges) | {int(x) for x in extra})


def test_dense_prefill_full_sampled_rows(dsa):
    """32768 causal rows x 32768 keys, 64 heads, k 2048 (rows shorter than k
    return every key); the edge rows and 248 seeded rows across the triangle."""
    wl = datagen.WORKLOADS[3]
    say("[full] dense prefill 32768 x 32768")
    dev, h = _device_inputs(wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], None,
                                      top_k=wl.top_k)
    rows = _prefill_rows([0, 1, 2046, 2047, 2048, 5000, 16383, 32767], seed=31)
    gi, gv = idx[rows].cpu().numpy(), val[rows].cpu().numpy()
    K = O.to_f64(datagen.keys(wl, 0, h["q"], h["w"]), wl.dtype)

    def row(i):
        t = rows[i]
        q_t, w_t = O.to_f64(h["q"][t], wl.dtype), h["w"][t].astype(np.float64)
        r = O.dense_row(q_t, w_t, K, t, wl.top_k)
        return _check(gi[i], gv[i], r, wl.top_k, q_t, w_t, K, f"row {t}")

    errs = _rows_parallel(row, range(len(rows)))
    assert not errs, "\n".join(errs[:10])


def test_misa_prefill_full_sampled_rows(dsa):
    """MISA on the prefill geometry at full size: the dense prefill workload's
    32768 rows x 32768 keys, 64 heads, routed to h = 8 over 64-key pooled
    blocks, k 2048; the edge rows and 248 seeded rows, each checked on its
    routed heads and then on the selection given the GPU's heads."""
    wl = datagen.WORKLOADS[3]
    h, B = 8, 64
    say("[full] MISA prefill 32768 x 32768, h 8")
    dev, hin = _device_inputs(wl)
    res = dsa.misa_route_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], None, block=B,
                                    n_active_heads=h, top_k=wl.top_k, with_importance=True)
    rows = _prefill_rows([0, 63, 64, 2047, 2048, 9999, 32767], seed=32)
    gi = res["idx"][rows].cpu().numpy()
    gv = res["score"][rows].cpu().numpy()
    gh = res["heads"][rows].cpu().numpy().astype(np.int64)
    gI = res["importance"][rows].cpu().numpy().astype(np.float64)
    K = O.to_f64(datagen.keys(wl, 0, hin["q"], hin["w"]), wl.dtype)

    def row(i):
        t = rows[i]
        errs = []
        q_t, w_t = O.to_f64(hin["q"][t], wl.dtype), hin["w"][t].astype(np.float64)
        pooled = O.misa_pooled_for_query(K, B, t)
        I = O.misa_importance(q_t, w_t, pooled)
        Fi = np.abs(w_t) * (np.abs(q_t) @ np.abs(pooled).T).sum(axis=1)
        bad = ~scores_ok(gI[i], I, I, Fi)
        if bad.any():
            errs.append(f"importance row {t}: {np.nonzero(bad)[0][:4]}")
        errs += check_selection(gh[i], None, np.arange(wl.n_heads), I, I, h, Fi,
                                what=f"heads row {t}")
        r = O.misa_row(q_t, w_t, K, t, B, h, wl.top_k, heads=gh[i])
        errs += _check(gi[i], gv[i], r, wl.top_k, q_t, w_t, K, f"misa row {t}", gh[i])
        return errs

    errs = _rows_parallel(row, range(len(rows)))
    assert not errs, "\n".join(errs[:10])


def test_hisa_prefill_full_sampled_rows(dsa):
    """HISA on the prefill geometry at full size: 32768 rows x 32768 keys, 64
    heads, 128-key blocks, m 64, k 2048; the edge rows (short rows that keep
    every block, rows whose last block is partial, the longest row) and 248
    seeded rows, each checked on its block selection and then on the token
    selection inside the GPU's blocks."""
    wl = datagen.WORKLOADS[3]
    B, m = 128, 64
    say("[full] HISA prefill 32768 x 32768, B 128, m 64")
    dev, hin = _device_inputs(wl)
    res = dsa.hisa_block_filter_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], None, block=B,
                                     m_blocks=m, top_k=wl.top_k)
    rows = _prefill_rows([0, 127, 2047, 8191, 8192, 20000, 32767], seed=33)
    gi = res["idx"][rows].cpu().numpy()
    gv = res["score"][rows].cpu().numpy()
    gb = res["blocks"][rows].cpu().numpy()
    gbs = res["block_score"][rows].cpu().numpy()
    K = O.to_f64(datagen.keys(wl, 0, hin["q"], hin["w"]), wl.dtype)

    def row(i):
        t = rows[i]
        q_t, w_t = O.to_f64(hin["q"][t], wl.dtype), hin["w"][t].astype(np.float64)
        pooled = O.misa_pooled_for_query(K, B, t)
        bs, bA = O.hisa_block_scores(q_t, w_t, pooled)
        Fb = O.dot_magnitude(q_t, w_t, pooled)
        errs = check_selection(gb[i], gbs[i], np.arange(pooled.shape[0]), bs, bA, m, Fb,
                               what=f"blocks row {t}")
        r = O.hisa_row(q_t, w_t, K, t, B, m, wl.top_k, blocks=gb[i])
        return errs + _check(gi[i], gv[i], r, wl.top_k, q_t, w_t, K, f"hisa row {t}")

    errs = _rows_parallel(row, range(len(rows)))
    assert not errs, "\n".join(errs[:10])
