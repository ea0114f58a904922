"""GPU parity of the dense indexer, pooling and IoU against the CPU oracle."""
import numpy as np
import pytest
import torch

import datagen
from oracle import indexer as O
from oracle.check import check_exact

from _helpers import check_rows, dense_ref, say, to_device, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_indexer_amd as m
    m.lib()  # fails loudly if the library is not built
    return m


def _run_dense(dsa, wl, seed=0, rows=None, k=None):
    k = k or wl.top_k
    inp = datagen.make(wl, seed)
    say(f"[dense] {wl.name} nq={wl.nq} L={wl.l_max} H={wl.n_heads} d={wl.head_dim} "
        f"{wl.dtype} k={k} seed={seed}")
    dev = upload(inp, wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=k)
    torch.cuda.synchronize()
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    rows = range(wl.nq) if rows is None else rows
    ref, qwk = dense_ref(inp, wl, rows, k)
    errs = check_rows(gi, gv, ref, k, qwk)
    assert not errs, "\n".join(errs[:10])
    return inp, gi, gv


def test_tiny_f32_workload(dsa):
    """The tiny float32 workload at full size (16 queries at the end of a 4096-key
    cache, 8 heads, d = 64, k = 64)."""
    _run_dense(dsa, datagen.WORKLOADS[1])


def test_tiny_workload_in_bf16_and_more_heads(dsa):
    for H, d in ((8, 64), (16, 128), (32, 128), (48, 64), (64, 128), (3, 128)):
        wl = datagen.WORKLOADS[1].replace(dtype=datagen.BF16, n_heads=H, head_dim=d)
        _run_dense(dsa, wl)
    _run_dense(dsa, datagen.WORKLOADS[1].replace(n_heads=3, head_dim=128))   # f32, odd H


def test_decode_many_chunks_ragged(dsa):
    """64 sequences of 70001 keys: 9 chunks of 8192 per query with a ragged tail."""
    wl = datagen.small(2, nq=64, n_seq=64, l_max=70001)
    _run_dense(dsa, wl, rows=range(0, 64, 3))


def test_decode_small_chunks(dsa):
    """Few queries with prefixes longer than a short pass (16384 items), so the
    library splits each prefix into many 256-key chunks."""
    wl = datagen.small(2, nq=4, n_seq=4, l_max=20000)
    _run_dense(dsa, wl)


def test_short_pass_switch_point(dsa):
    """16384 keys per query go through the short pass (every (key, id) stored,
    one workgroup per query selects); 16385 through the chunked pass with the
    merge.  Both against the oracle, with a prefix shorter than k as well."""
    for L in (16384, 16385):
        wl = datagen.small(2, nq=6, n_seq=6, l_max=L)
        inp = datagen.make(wl, 7)
        inp["q_pos"] = np.array([L - 1, L - 2, 9000, 2047, 100, 0], dtype=np.int32)
        say(f"[dense] switch point L={L}")
        dev = upload(inp, wl)
        idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                          top_k=2048)
        ref, qwk = dense_ref(inp, wl, range(6), 2048)
        errs = check_rows(idx.cpu().numpy(), val.cpu().numpy(), ref, 2048, qwk)
        assert not errs, "\n".join(errs[:10])


def test_short_prefixes_and_padding(dsa):
    """Queries on one shared cache at positions 0 .. 5000 with k = 2048: rows
    shorter than k return every key and pad with (-1, -inf)."""
    wl = datagen.small(2, nq=8, n_seq=1, l_max=6000, layout="tail", plant="points", n_plant=40)
    inp = datagen.make(wl, 3)
    inp["q_pos"] = np.array([0, 1, 5, 100, 2046, 2047, 2048, 5000], dtype=np.int32)
    dev = upload(inp, wl)
    say("[dense] short prefixes")
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=2048)
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    ref, qwk = dense_ref(inp, wl, range(8), 2048)
    errs = check_rows(gi, gv, ref, 2048, qwk)
    assert not errs, "\n".join(errs[:10])
    assert sorted(gi[0, :1].tolist()) == [0] and np.all(gi[0, 1:] == -1)
    assert np.all(np.isneginf(gv[3, 101:]))


def test_top1_and_topk_larger_than_cache(dsa):
    wl = datagen.small(2, nq=4, n_seq=4, l_max=3000)
    for k in (1, 7, 4000):
        _run_dense(dsa, wl, k=k)


def test_all_equal_keys_pin_the_tie_break(dsa):
    """Every key identical: all scores tie, so the selection must be exactly the
    k lowest indices.  70000 keys in 64 queries' caches also force the merge's
    fallback path (the tied bin does not fit in LDS)."""
    for nq, L, k in ((4, 5000, 100), (64, 70000, 2048)):
        wl = datagen.small(2, nq=nq, n_seq=nq, l_max=L)
        inp = datagen.make(wl, 1)
        inp["k"][:] = inp["k"][:, :1, :]
        say(f"[dense] all-equal keys nq={nq} L={L} k={k}")
        dev = upload(inp, wl)
        idx, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                        top_k=k)
        gi = idx.cpu().numpy()
        for t in range(nq):
            assert check_exact(gi[t], np.arange(k)) == [], f"query {t}"


def test_keys_sorted_by_increasing_score(dsa):
    """Keys reordered so the score grows with the position (winners come last)."""
    wl = datagen.small(2, nq=2, n_seq=2, l_max=20000)
    inp = datagen.make(wl, 5)
    for t in range(2):
        q_t = O.to_f64(inp["q"][t], wl.dtype)
        K = O.to_f64(inp["k"][t], wl.dtype)
        s, _ = O.indexer_scores(q_t, inp["w"][t].astype(np.float64), K)
        inp["k"][t] = inp["k"][t][np.argsort(s, kind="stable")]
    say("[dense] sorted keys")
    dev = upload(inp, wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=2048)
    ref, qwk = dense_ref(inp, wl, range(2), 2048)
    errs = check_rows(idx.cpu().numpy(), val.cpu().numpy(), ref, 2048, qwk)
    assert not errs, "\n".join(errs[:10])


def test_negative_weights_ties_at_zero(dsa):
    """All weights negative: every score is <= 0 and the winners are the keys
    with no positive head dot (score exactly 0), ranked by index."""
    wl = datagen.small(2, nq=4, n_seq=4, l_max=5000, n_heads=8)
    inp = datagen.make(wl, 6)
    inp["w"] = -np.abs(inp["w"])
    _ = upload(inp, wl)
    say("[dense] negative weights")
    dev = upload(inp, wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=64)
    ref, qwk = dense_ref(inp, wl, range(4), 64)
    errs = check_rows(idx.cpu().numpy(), val.cpu().numpy(), ref, 64, qwk)
    assert not errs, "\n".join(errs[:10])


def test_invalid_rows_are_padding(dsa):
    wl = datagen.small(2, nq=4, n_seq=2, l_max=1000, layout="tail", plant="points", n_plant=0)
    inp = datagen.make(wl, 0)
    inp["q_seq"] = np.array([0, 5, -1, 1], dtype=np.int32)
    inp["q_pos"] = np.array([-3, 10, 10, 1000], dtype=np.int32)
    dev = upload(inp, wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=16)
    assert np.all(idx.cpu().numpy() == -1)
    assert np.all(np.isneginf(val.cpu().numpy()))


def test_repeat_calls_same_sets(dsa):
    wl = datagen.small(2, nq=16, n_seq=16, l_max=30000)
    inp = datagen.make(wl, 7)
    dev = upload(inp, wl)
    a, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"], top_k=512)
    b, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"], top_k=512)
    assert torch.equal(torch.sort(a, 1).values, torch.sort(b, 1).values)


def test_argument_errors(dsa):
    wl = datagen.small(2, nq=2, n_seq=2, l_max=100)
    dev = upload(datagen.make(wl, 0), wl)
    with pytest.raises(dsa.DsaError):
        dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"], top_k=0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises((dsa.DsaError, ValueError)):
        dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"], top_k=8,
                               workspace=ws)


def test_mean_pool_matches_oracle_bits(dsa):
    for L, B, d in ((4096, 64, 128), (1000, 128, 128), (777, 7, 64), (130, 1, 128)):
        wl = datagen.small(4, nq=3, n_seq=3, l_max=L, head_dim=d, block=B)
        inp = datagen.make(wl, 2)
        say(f"[pool] L={L} B={B} d={d}")
        k = to_device(inp["k"], wl.dtype)
        got = dsa.indexer_mean_pool_keys(k, B).view(torch.int16).cpu().numpy().view(np.uint16)
        for s in range(3):
            ref = O.f64_to_bf16_bits(O.pooled_cache(O.to_f64(inp["k"][s], wl.dtype), B))
            assert np.array_equal(got[s], ref), f"seq {s}: {(got[s] != ref).sum()} bf16 values differ"


def test_iou_kernel(dsa):
    rng = np.random.default_rng(0)
    nq, k = 20, 300
    A = np.stack([rng.permutation(1000)[:k] for _ in range(nq)]).astype(np.int32)
    B = np.stack([rng.permutation(1000)[:k] for _ in range(nq)]).astype(np.int32)
    A[3, 100:] = -1
    B[4, :] = -1
    A[5, :] = -1; B[5, :] = -1
    B[6] = A[6][::-1]
    got = dsa.indexer_selection_iou(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()).cpu().numpy()
    ref = O.iou_rows(A, B)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=0)
    assert got[5] == 1.0 and got[6] == 1.0 and got[4] == 0.0
