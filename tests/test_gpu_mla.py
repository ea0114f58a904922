"""GPU parity of the sparse attention over the selected index list.

Every checked output value must satisfy
    |o_gpu - o| <= 2^-7 * sum_i p_i |v_i| + 2^-8 * |o|
with o and the weights p from the float64 oracle.  The kernel's own error:
bf16 rounding of each probability before the value product (relative 2^-9
per term, so at most 2^-9 * sum_i p_i |v_i| over the row, and the same again
for the sum in the denominator, which is kept unrounded), float32 scores and
accumulation (relative ~2^-20), the bf16 rounding of each slice's output when
a list is split over workgroups (at most 2^-9 * sum_i p_i |v_i| after the
merge) and of the output (2^-9 |o|): 2^-8 * sum_i p_i |v_i| + 2^-9 |o| in
all.  The bound above leaves a factor of two over that.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import datagen
from datagen import mla as M
from oracle import attention as A

from _helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_indexer_amd as m
    m.lib()
    return m


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def _f64(bits: np.ndarray) -> np.ndarray:
    return datagen.bf16_bits_to_f32(bits).astype(np.float64)


def _check_rows(o, q, rows_of, idx, qs, qp, wl, rows, what):
    errs = []
    for t in rows:
        kv_rows = rows_of(int(qs[t]), int(qp[t]))
        ref, mag = A.sparse_mla_row(_f64(q[t]), kv_rows, idx[t], wl.d_v, wl.scale)
        bad = np.abs(o[t] - ref) > 2.0 ** -7 * mag + 2.0 ** -8 * np.abs(ref)
        if bad.any():
            h, c = np.argwhere(bad)[0]
            errs.append(f"{what} q{t}: {int(bad.sum())} values off, first head {h} col {c}: "
                        f"gpu {o[t, h, c]} ref {ref[h, c]} mag {mag[h, c]}")
    assert not errs, "\n".join(errs[:8])


def _case(dsa, wl, seed=0, idx=None, qs=None, qp=None, rows=None, what="mla"):
    q = M.queries(wl, seed)
    C = M.cache(wl, seed)
    qs0, qp0 = M.positions(wl)
    qs = qs0 if qs is None else np.asarray(qs, dtype=np.int32)
    qp = qp0 if qp is None else np.asarray(qp, dtype=np.int32)
    idx = M.index_lists(wl, seed) if idx is None else np.asarray(idx, dtype=np.int32)
    say(f"[{what}] nq={wl.nq} L={wl.l_max} H={wl.n_heads} k={idx.shape[1]} "
        f"ws={dsa.sparse_mla_workspace_size(wl.nq, wl.n_heads, wl.d_qk, wl.d_v, idx.shape[1])}")
    out = dsa.sparse_mla_attention(_bf16(q), _bf16(C), torch.from_numpy(qp).cuda(),
                                   torch.from_numpy(idx).cuda(), torch.from_numpy(qs).cuda(),
                                   softmax_scale=wl.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)

    def rows_of(s, p):
        if not (0 <= s < wl.n_seq and 0 <= p < wl.l_max):
            return np.zeros((0, wl.d_qk))
        return _f64(C[s, :p + 1])
    _check_rows(o, q, rows_of, idx, qs, qp, wl, range(wl.nq) if rows is None else rows, what)
    return o


def test_mla_split_lists_all_head_counts(dsa):
    """Lists split over several workgroups (few queries): 32..128 heads."""
    for H in (128, 32, 64, 96):
        wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(
            nq=8, n_seq=1, l_max=3000, n_heads=H, top_k=2048, layout="tail")
        _case(dsa, wl, seed=H, what=f"mla H{H}")


def test_mla_unsplit_lists_and_ragged_k(dsa):
    """Enough queries that every list stays in one workgroup; k not a multiple
    of the 32-row step."""
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(
        nq=320, n_seq=1, l_max=2000, n_heads=64, top_k=1000, layout="tail")
    _case(dsa, wl, seed=3, rows=list(range(0, 320, 29)) + [319])
    wl = wl.replace(nq=16, top_k=77)
    _case(dsa, wl, seed=4)


def test_mla_padding_repeats_out_of_range_and_invalid_rows(dsa):
    """-1 padding (prefixes shorter than k), entries beyond the prefix or the
    cache, repeated entries, and queries with no keys at all."""
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(
        nq=12, n_seq=2, l_max=100, n_heads=128, top_k=160, layout="tail")
    qs = np.array([0, 1] * 6, dtype=np.int32)
    qp = np.array([0, 5, 31, 32, 63, 99, 99, 50, -1, 100, 99, 7], dtype=np.int32)
    idx = np.full((12, 160), -1, dtype=np.int32)
    rng = np.random.default_rng(7)
    for t in range(12):
        n = max(int(qp[t]) + 1, 1)
        idx[t, :min(n, 160)] = rng.permutation(n)[:160]
    idx[6, 100:140] = rng.integers(0, 100, size=40)           # repeats
    idx[7, 60:70] = [51, 60, 99, 100, 5000, -7, 50, 0, 50, 2]  # beyond the prefix / cache
    qs_bad = qs.copy()
    qs_bad[10] = 5                                             # no such cache
    _case(dsa, wl, seed=5, idx=idx, qs=qs_bad, qp=qp, what="mla edge")


def test_mla_after_the_indexer(dsa):
    """The dense indexer's top-k (with its padding) fed straight to the
    attention over a latent cache of the same length."""
    iwl = datagen.small(2, nq=8, n_seq=8, l_max=4096)
    inp = datagen.make(iwl, 0)
    from _helpers import upload
    dev = upload(inp, iwl)
    sel, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    top_k=2048)
    idx = sel.cpu().numpy()
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(nq=8, n_seq=8, l_max=4096)
    _case(dsa, wl, seed=6, idx=idx, what="mla after indexer")


def test_mla_score_far_above_the_first_steps(dsa):
    """A listed row whose score for some heads exceeds everything before it
    in its slice by far more than the kernel's fixed softmax reference allows
    (the row is 8 times one head's query row, a score near 8 |q|^2), placed
    after the first step of its slice: the kernel redoes the slice with the
    slice's largest score as the reference, and the result must meet the same
    bound against the oracle."""
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(
        nq=4, n_seq=1, l_max=4096, n_heads=128, top_k=2048, layout="tail")
    q = M.queries(wl, 11)
    C = M.cache(wl, 11).copy()
    qs, qp = M.positions(wl)
    idx = M.index_lists(wl, 11)
    qf = datagen.bf16_bits_to_f32(q)
    # entries 100 and 1500: step 3 of the first 128-entry slice and step 2 of
    # the twelfth (the call splits each list into 16 slices of 4 steps)
    for t in range(wl.nq):
        for j, h in ((100, 5), (1500, 77)):
            C[int(qs[t]), int(idx[t, j])] = datagen.f32_to_bf16_bits(8.0 * qf[t, h])
    say(f"[mla far scores] nq={wl.nq} L={wl.l_max} H={wl.n_heads} k={wl.top_k}")
    out = dsa.sparse_mla_attention(_bf16(q), _bf16(C), torch.from_numpy(qp).cuda(),
                                   torch.from_numpy(idx).cuda(), torch.from_numpy(qs).cuda(),
                                   softmax_scale=wl.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    _check_rows(o, q, lambda s, p: _f64(C[s, :p + 1]), idx, qs, qp, wl, range(wl.nq),
                "mla far scores")
    # the planted heads attend almost only to their row
    for t in range(wl.nq):
        for j, h in ((100, 5), (1500, 77)):
            row = _f64(C[int(qs[t]), int(idx[t, j])])[:wl.d_v]
            assert np.abs(o[t, h] - row).max() < 2.0 ** -6 * np.abs(row).max() + 1e-3


def test_mla_full_size_every_query(dsa):
    """64 queries x 128 heads over their own 131072-row caches, k = 2048, as
    timed: the rows the lists name are generated and placed in a zeroed cache
    (no other row is read), and every query is checked against the oracle."""
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"]
    q = M.queries(wl, 0)
    idx = M.index_lists(wl, 0)
    qs, qp = M.positions(wl)
    say(f"[mla full] nq={wl.nq} L={wl.l_max} H={wl.n_heads} k={wl.top_k}")
    kv = torch.zeros((wl.n_seq, wl.l_max, wl.d_qk), dtype=torch.bfloat16, device="cuda")
    gathered = {}
    for t in range(wl.nq):
        r = M.rows(wl, int(qs[t]), idx[t], 0)
        gathered[t] = r
        kv[int(qs[t])][torch.from_numpy(idx[t].astype(np.int64)).cuda()] = _bf16(r)
    out = dsa.sparse_mla_attention(_bf16(q), kv, torch.from_numpy(qp).cuda(),
                                   torch.from_numpy(idx).cuda(), torch.from_numpy(qs).cuda(),
                                   softmax_scale=wl.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    del kv
    def check(t):
        ref, mag = A.sparse_mla_row(_f64(q[t]), _f64(gathered[t]), np.arange(wl.top_k), wl.d_v,
                                    wl.scale)
        bad = np.abs(o[t] - ref) > 2.0 ** -7 * mag + 2.0 ** -8 * np.abs(ref)
        return [f"q{t}: {int(bad.sum())} values off"] if bad.any() else []

    # (the oracle's NumPy work releases the interpreter lock)
    with ThreadPoolExecutor(max_workers=16) as ex:
        errs = [e for es in ex.map(check, range(wl.nq)) for e in es]
    assert not errs, "\n".join(errs)


def test_mla_argument_errors(dsa):
    """Calls the library rejects before any launch."""
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(nq=2, n_seq=2, l_max=64, n_heads=32,
                                                             top_k=16)
    q = _bf16(M.queries(wl, 0))
    kv = _bf16(M.cache(wl, 0))
    qs, qp = (torch.from_numpy(x).cuda() for x in M.positions(wl))
    idx = torch.from_numpy(M.index_lists(wl, 0)).cuda()
    for bad in (0.0, float("nan"), -1.0, float("inf")):
        with pytest.raises(dsa.DsaError):
            dsa.sparse_mla_attention(q, kv, qp, idx, qs, softmax_scale=bad)
    q48 = torch.zeros((2, 48, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DsaError):                       # 48 heads: not a multiple of 32
        dsa.sparse_mla_attention(q48, kv, qp, idx, qs, softmax_scale=0.1)
    q512 = torch.zeros((2, 32, 512), dtype=torch.bfloat16, device="cuda")
    kv512 = torch.zeros((2, 64, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DsaError):                       # rows of 512: not the 576 layout
        dsa.sparse_mla_attention(q512, kv512, qp, idx, qs, softmax_scale=0.1)
    big = torch.zeros((2, 32769), dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError):                       # list longer than supported
        dsa.sparse_mla_attention(q, kv, qp, big, qs, softmax_scale=0.1)
    idx256 = torch.full((2, 256), -1, dtype=torch.int32, device="cuda")
    idx256[:, :16] = idx
    need = dsa.sparse_mla_workspace_size(2, 32, 576, 512, 256)
    assert need > 0                                         # two queries: lists are split
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises((dsa.DsaError, ValueError)):
        dsa.sparse_mla_attention(q, kv, qp, idx256, qs, softmax_scale=0.1, workspace=ws)


def test_mla_without_sequence_ids(dsa):
    """q_seq omitted: every query reads cache 0."""
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(
        nq=5, n_seq=1, l_max=700, n_heads=64, top_k=300, layout="tail")
    q = M.queries(wl, 9)
    C = M.cache(wl, 9)
    _, qp = M.positions(wl)
    idx = M.index_lists(wl, 9)
    out = dsa.sparse_mla_attention(_bf16(q), _bf16(C), torch.from_numpy(qp).cuda(),
                                   torch.from_numpy(idx).cuda(), None, softmax_scale=wl.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    _check_rows(o, q, lambda s, p: _f64(C[0, :p + 1]), idx, np.zeros(5, np.int32), qp, wl,
                range(5), "mla no q_seq")
