"""GPU parity of the prefill-shaped path (many query rows on one sequence)."""
import numpy as np
import pytest
import torch

import datagen
from oracle import indexer as O
from oracle.check import check_exact

from _helpers import check_rows, dense_ref, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_indexer_amd as m
    m.lib()
    return m


def _run(dsa, wl, k, seed=0, pos=None, seq=None, rows=None):
    inp = datagen.make(wl, seed)
    if pos is not None:
        inp["q_pos"] = np.asarray(pos, dtype=np.int32)
    if seq is not None:
        inp["q_seq"] = np.asarray(seq, dtype=np.int32)
    say(f"[prefill] nq={wl.nq} L={wl.l_max} H={wl.n_heads} d={wl.head_dim} k={k} seed={seed}")
    dev = upload(inp, wl)
    idx, val = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                      top_k=k)
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    rows = range(wl.nq) if rows is None else rows
    valid = [t for t in rows if inp["q_seq"][t] == 0 and 0 <= inp["q_pos"][t] < wl.l_max]
    ref, qwk = dense_ref(inp, wl, valid, k)
    errs = check_rows(gi, gv, ref, k, qwk)
    for t in rows:
        if t not in valid:
            assert np.all(gi[t] == -1) and np.all(np.isneginf(gv[t])), f"invalid row {t}"
    assert not errs, "\n".join(errs[:10])
    return inp, gi, gv


def test_prefill_rows(dsa):
    """512 causal rows of a 512-key cache (ragged last stage), k = 64: rows
    0..62 are shorter than k and return every key."""
    wl = datagen.small(3, nq=512, l_max=512, n_plant=16)
    _run(dsa, wl, 64)


def test_prefill_rows_larger(dsa):
    wl = datagen.small(3, nq=2048, l_max=2048, n_plant=64)
    _run(dsa, wl, 300, seed=1, rows=list(range(0, 2048, 37)) + [2047])


def test_prefill_heads_and_dims(dsa):
    for H, d in ((32, 128), (64, 64), (16, 128), (48, 128)):
        wl = datagen.small(3, nq=256, l_max=700, n_heads=H, head_dim=d, n_plant=8)
        _run(dsa, wl, 100, seed=2)


def test_prefill_arbitrary_positions_and_invalid_rows(dsa):
    """Positions in any order, repeated positions, and rows that are not valid
    for a one-sequence call (sequence id 1, negative or too large positions)."""
    wl = datagen.small(3, nq=100, l_max=3000, n_plant=16)
    rng = np.random.default_rng(3)
    pos = rng.integers(0, 3000, size=100)
    pos[5] = -1
    pos[6] = 3000
    pos[7] = 2999
    pos[8] = 0
    seq = np.zeros(100, dtype=np.int32)
    seq[9] = 1
    _run(dsa, wl, 256, seed=4, pos=pos, seq=seq)


def test_prefill_all_equal_keys(dsa):
    """All scores tie: rows select exactly their lowest indices; 20000-key rows
    overflow the LDS list and use the global fallback."""
    wl = datagen.small(3, nq=64, l_max=20000, layout="tail", n_plant=0)
    inp = datagen.make(wl, 5)
    inp["k"][:] = inp["k"][:, :1, :]
    dev = upload(inp, wl)
    idx, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    top_k=2048)
    gi = idx.cpu().numpy()
    for t in range(64):
        assert check_exact(gi[t], np.arange(2048)) == [], f"row {t}"


def test_shared_cache_decode_queries_long_rows(dsa):
    """64 decode queries sharing one 131072-key cache (its last 64 positions),
    64 heads, k 2048: the query-grouped kernels with 11-bit bins and 32-bit
    per-row counters (rows longer than 65535 keys); every row."""
    wl = datagen.small(2, nq=64, n_seq=1, l_max=131072, layout="tail")
    _run(dsa, wl, 2048, seed=6)


def test_long_prefill_chunk_arbitrary_positions(dsa):
    """A chunk of 96 prefill rows at arbitrary positions of one 100000-key
    cache (32 heads, d 64, k 1000), with invalid rows and rows shorter than k;
    sampled rows plus the invalid ones."""
    wl = datagen.small(3, nq=96, l_max=100000, n_heads=32, head_dim=64, n_plant=64)
    rng = np.random.default_rng(8)
    pos = rng.integers(0, 100000, size=96)
    pos[0], pos[1], pos[2], pos[3] = 99999, 65534, 65535, 500
    pos[4] = -1
    seq = np.zeros(96, dtype=np.int32)
    seq[5] = 1
    _run(dsa, wl, 1000, seed=7, pos=pos, seq=seq, rows=list(range(0, 96, 7)) + [1, 2, 3, 4, 5])


def test_key_split_rows_at_part_boundaries(dsa):
    """24 rows of one 70000-key cache: 3 row groups, so the keys are split over
    workgroups and the row select works in parts of 8192 keys.  Rows end
    exactly at, just past and just before part boundaries, at and just past
    k, and on a single key; every row."""
    wl = datagen.small(3, nq=24, l_max=70000, n_heads=16, head_dim=64, n_plant=32)
    k = 1500
    pos = [8191, 8192, 8190, 16383, 16384, 24575, 24576, 65535, 65536, 69999, k - 1, k,
           k - 2, 0, 40959, 40960, 57343, 57344, 12345, 33333, 49151, 49152, 1, 69998]
    _run(dsa, wl, k, seed=12, pos=pos)


def test_long_rows_all_equal_keys(dsa):
    """All scores tie in 70000-key rows (11-bit bins, the tie bin overflows
    LDS): the lowest indices are selected."""
    wl = datagen.small(3, nq=64, l_max=70000, layout="tail", n_plant=0)
    inp = datagen.make(wl, 9)
    inp["k"][:] = inp["k"][:, :1, :]
    dev = upload(inp, wl)
    idx, _ = dsa.indexer_score_topk(dev["q"], dev["w"], dev["k"], dev["q_pos"], dev["q_seq"],
                                    top_k=2048)
    gi = idx.cpu().numpy()
    for t in range(64):
        assert check_exact(gi[t], np.arange(2048)) == [], f"row {t}"


def test_long_rows_many_row_groups(dsa):
    """2048 rows (256 row groups: no key split) at arbitrary positions of one
    70000-key cache: rows longer than 65535 keys use 11-bit bins with 32-bit
    per-row counters in the scoring kernel; sampled rows."""
    wl = datagen.small(3, nq=2048, l_max=70000, n_heads=16, head_dim=64, n_plant=64)
    rng = np.random.default_rng(10)
    pos = rng.integers(0, 70000, size=2048)
    pos[:8] = [69999, 65535, 65534, 2047, 2048, 0, 69998, 40000]
    _run(dsa, wl, 2048, seed=11, pos=pos, rows=list(range(0, 2048, 97)) + list(range(8)))
