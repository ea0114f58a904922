"""Certified exact top-k (the DoSA review's screen / bound / prune / rescore,
sections 1 and 3; bounds from Cauchy-Schwarz): on the GPU, through the C ABI.

The call's result must be the dense call's exactly: the survivors are
rescored with every head as the dense call scores them, so every (index,
score) pair agrees bit for bit.  Its survivor counts must cover the oracle's
certificate (the GPU bounds are the oracle's widened by a rounding margin, so
the GPU keeps at least every key the exact certificate keeps), and the oracle's
exact top-k must pass the usual selection check against the call's output.

Inputs: the dense workloads' seeded generators, plus a "concentrated weights"
recipe (seeded numpy): 8 heads with w ~ N(0, 1), the other heads' weights
scaled by 1e-3, q and k ~ N(0, 1) rounded to bf16 - the case where the bounds
of the heads left out are tight enough to prune.
"""
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


def _same_as_dense(ci, cs, di, ds, what):
    errs = []
    for t in range(ci.shape[0]):
        a = {int(i): s for i, s in zip(ci[t], cs[t].view(np.uint32)) if i >= 0}
        b = {int(i): s for i, s in zip(di[t], ds[t].view(np.uint32)) if i >= 0}
        if a != b:
            errs.append(f"{what} q{t}: {len(set(a) ^ set(b))} indices differ, "
                        f"{sum(a[i] != b[i] for i in set(a) & set(b))} scores differ")
        if (ci[t] < 0).sum() != (di[t] < 0).sum():
            errs.append(f"{what} q{t}: padding differs")
    return errs


def _run_both(dsa, dev, k, h):
    res = dsa.indexer_certified_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                     top_k=k, n_screen_heads=h)
    di, ds = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    top_k=k)
    torch.cuda.synchronize()
    return ({key: v.cpu().numpy() for key, v in res.items()}, di.cpu().numpy(), ds.cpu().numpy())


def _oracle_checks(inp, wl, out, k, h, rows):
    errs = []
    for t in rows:
        s = int(inp["q_seq"][t])
        q_t = O.to_f64(inp["q"][t], wl.dtype)
        w_t = inp["w"][t].astype(np.float64)
        K = O.to_f64(inp["k"][s], wl.dtype)
        p = int(inp["q_pos"][t])
        if p < 0:
            if out["survivors"][t] != 0:
                errs.append(f"q{t}: invalid query with {out['survivors'][t]} survivors")
            continue
        c = O.dosa_certificate(q_t, w_t, K[:p + 1], k, h)
        if out["survivors"][t] < int(c["survive"].sum()):
            errs.append(f"q{t}: {out['survivors'][t]} survivors < the certificate's "
                        f"{int(c['survive'].sum())}")
        d = O.dense_row(q_t, w_t, K, p, k)
        F = O.dot_magnitude(q_t, w_t, K[d["cand"]])
        errs += check_selection(out["idx"][t], out["score"][t], d["cand"], d["s"], d["A"], k, F,
                                what=f"certified q{t}")
    return errs


def test_certified_equals_dense_reduced(dsa):
    wl = datagen.small(2, nq=8, n_seq=8, l_max=32768, n_plant=64)
    inp = datagen.make(wl, 3)
    say(f"[certified] nq={wl.nq} L={wl.l_max} H={wl.n_heads} k={wl.top_k}")
    dev = upload(inp, wl)
    for h in (4, 16):
        out, di, ds = _run_both(dsa, dev, wl.top_k, h)
        errs = _same_as_dense(out["idx"], out["score"], di, ds, f"h={h}")
        errs += _oracle_checks(inp, wl, out, wl.top_k, h, rows=range(wl.nq))
        assert not errs, "\n".join(errs[:12])


def _concentrated(nq, n_seq, L, H, D, seed):
    rng = np.random.default_rng(seed)
    to_bf16 = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    q = to_bf16(rng.standard_normal((nq, H, D)))
    w = rng.standard_normal((nq, H)).astype(np.float32)
    w[:, 8:] *= 1e-3
    k = to_bf16(rng.standard_normal((n_seq, L, D)))
    bits = lambda x: x.view(torch.int16).numpy().view(np.uint16)
    inp = {"q": bits(q), "w": w, "k": bits(k), "q_seq": np.arange(nq, dtype=np.int32) % n_seq,
           "q_pos": np.full(nq, L - 1, dtype=np.int32)}
    dev = {"q": q.cuda(), "w": torch.from_numpy(w).cuda(), "k": k.cuda(),
           "q_seq": torch.from_numpy(inp["q_seq"]).cuda(),
           "q_pos": torch.from_numpy(inp["q_pos"]).cuda()}
    return inp, dev


def test_certified_prunes_with_concentrated_weights(dsa):
    nq, n_seq, L, H, D, k = 8, 8, 65536, 64, 128, 512
    say(f"[certified concentrated] nq={nq} L={L} H={H} k={k}")
    inp, dev = _concentrated(nq, n_seq, L, H, D, 5)
    wl = datagen.small(2, nq=nq, n_seq=n_seq, l_max=L)
    out, di, ds = _run_both(dsa, dev, k, 8)
    errs = _same_as_dense(out["idx"], out["score"], di, ds, "concentrated")
    frac = out["survivors"] / L
    say(f"[certified concentrated] survivors per query {out['survivors'].tolist()} "
        f"(mean {frac.mean():.3f} of the keys)")
    if not (frac < 0.5).all():
        errs.append(f"expected pruning, survivors {out['survivors'].tolist()}")
    errs += _oracle_checks(inp, wl, out, k, 8, rows=range(nq))
    assert not errs, "\n".join(errs[:12])


def test_certified_short_and_invalid_rows(dsa):
    """Prefixes shorter than top_k keep every key (and pad), queries outside
    their cache give padding only; several queries share a cache."""
    wl = datagen.small(2, nq=12, n_seq=12, l_max=20000, n_plant=16)
    inp = datagen.make(wl, 7)
    inp["q_seq"] = (np.arange(12) % 3).astype(np.int32)      # three caches, four queries each
    inp["q_pos"] = np.array([0, 5, 100, 255, 256, 9999, 19999, -1, 20000, 3000, 12345, 1],
                            dtype=np.int32)
    say(f"[certified short] pos={inp['q_pos'].tolist()}")
    dev = upload(inp, wl)
    k = 256
    out, di, ds = _run_both(dsa, dev, k, 8)
    errs = _same_as_dense(out["idx"], out["score"], di, ds, "short")
    for t, p in enumerate(inp["q_pos"]):
        if 0 <= p < wl.l_max and p + 1 <= k and out["survivors"][t] != p + 1:
            errs.append(f"q{t}: pos {p}, {out['survivors'][t]} survivors (all {p + 1} expected)")
        if not (0 <= p < wl.l_max):
            if out["survivors"][t] != 0 or (out["idx"][t] != -1).any():
                errs.append(f"q{t}: invalid query not padded")
    ok = [t for t, p in enumerate(inp["q_pos"]) if 0 <= p < wl.l_max]
    inp_ok = dict(inp)
    errs += _oracle_checks(inp_ok, wl, out, k, 8, rows=ok)
    assert not errs, "\n".join(errs[:12])


def test_certified_full_dense_decode_workload(dsa):
    """64 queries x 131072 keys, 64 heads, k 2048, 16 screened heads: the
    dense call's result for every query; the oracle's certificate on sampled
    rows."""
    wl = datagen.WORKLOADS[2]
    inp = datagen.make(wl, 0)
    say(f"[certified full] nq={wl.nq} L={wl.l_max} H={wl.n_heads} k={wl.top_k}")
    dev = upload(inp, wl)
    out, di, ds = _run_both(dsa, dev, wl.top_k, 16)
    errs = _same_as_dense(out["idx"], out["score"], di, ds, "full")
    say(f"[certified full] survivors: mean {out['survivors'].mean() / wl.l_max:.4f} of the keys")
    errs += _oracle_checks(inp, wl, out, wl.top_k, 16, rows=(0, 31, 63))
    assert not errs, "\n".join(errs[:12])


def test_certified_argument_errors(dsa):
    wl = datagen.small(2, nq=2, n_seq=2, l_max=4096)
    inp = datagen.make(wl, 1)
    dev = upload(inp, wl)
    args = (dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"])
    for h in (0, 17, wl.n_heads + 1):
        with pytest.raises(dsa.DsaError):
            dsa.indexer_certified_topk(*args, top_k=64, n_screen_heads=h)
    with pytest.raises(dsa.DsaError):
        dsa.indexer_certified_topk(dev["q"].float(), dev["w"], dev["k"].float(), dev["q_pos"],
                                   dev["q_seq"], top_k=64, n_screen_heads=4)
