"""Seeded synthetic inputs for the DSA indexer workloads.

This module only draws inputs: query vectors ``q``, signed head weights ``w``,
the per-token indexer key cache ``K`` and the per-query (sequence, position)
pairs.  It contains none of the indexer's arithmetic (no scores, no selection,
no pooling), so both the CPU oracle and the GPU path may be fed from it.

Every random draw comes from ``numpy.random.default_rng(SeedSequence(...))``
keyed by ``(seed, workload id, purpose, sequence, chunk)``, so a sequence's
keys are the same bytes whether they are generated alone, in parallel, or all
at once.  bf16 tensors are carried as ``uint16`` bit patterns, rounded from
float32 draws by round-to-nearest-even.

Workload shapes follow the indexer settings the pages name: DeepSeek-V3.2's
64-head indexer and GLM-5's 32-head indexer (MISA summary, "problem" and
"results" sections), MISA's mean-pooled blocks with h=8 routed heads and a
k'=8192 candidate set (MISA summary, "method" and "hierarchical variant"), and
HISA's block filter with block size B and top-m blocks (HISA review, section 3).
The planted-key structure stands in for the real-model activations and
long-context suites the pages evaluate on, which are not available here: a
planted key is ``k[u] = q[t, j] + 0.3 * noise`` along one head's query vector.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

BF16 = "bf16"
F32 = "f32"

# purpose tags inside the SeedSequence key
_TAG_QUERY = 0
_TAG_PLANT = 1
_TAG_KEYS = 2

KEY_CHUNK = 65536  # keys per independently seeded generation chunk


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits.

    Generators only produce finite values, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic indexer workload.

    layout:
      ``"decode"``  query t runs against its own sequence t at position l_max-1
      ``"tail"``    one shared sequence; the queries sit at the last nq positions
      ``"prefill"`` one shared sequence; query row t sits at position t
    plant: which planted-key recipe to apply (see ``_plants``).
    """

    name: str
    wid: int
    nq: int
    n_seq: int
    l_max: int
    n_heads: int
    head_dim: int
    dtype: str
    top_k: int
    w_scale: float
    layout: str
    plant: str
    n_plant: int = 0          # recipe-dependent count (keys, or blocks)
    block: int = 0            # B (MISA / HISA)
    n_active_heads: int = 0   # h (MISA)
    k_prime: int = 0          # k' (MISA dagger)
    m_blocks: int = 0         # m (HISA)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def key_bytes(self) -> int:
        return self.head_dim * (2 if self.dtype == BF16 else 4)


# The five workloads.  ``wid`` is 1-based like the workload descriptions.
WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_dense_f32", 1, nq=16, n_seq=1, l_max=4096, n_heads=8, head_dim=64,
                dtype=F32, top_k=64, w_scale=1.0, layout="tail", plant="points", n_plant=32),
    2: Workload("dense_decode_L128K_H64", 2, nq=64, n_seq=64, l_max=131072, n_heads=64,
                head_dim=128, dtype=BF16, top_k=2048, w_scale=1.0 / 8.0, layout="decode",
                plant="fraction", n_plant=0),
    3: Workload("dense_prefill_L32K_H64", 3, nq=32768, n_seq=1, l_max=32768, n_heads=64,
                head_dim=128, dtype=BF16, top_k=2048, w_scale=1.0, layout="prefill",
                plant="points", n_plant=256),
    4: Workload("misa_decode_L128K_H64_h8", 4, nq=64, n_seq=64, l_max=131072, n_heads=64,
                head_dim=128, dtype=BF16, top_k=2048, w_scale=1.0, layout="decode",
                plant="hot_heads", n_plant=16, block=64, n_active_heads=8, k_prime=8192),
    5: Workload("hisa_decode_L1M_H32", 5, nq=32, n_seq=32, l_max=1048576, n_heads=32,
                head_dim=128, dtype=BF16, top_k=2048, w_scale=1.0, layout="decode",
                plant="blocks", n_plant=96, block=128, m_blocks=64),
}


def positions(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Per-query (sequence id, position) as int32 arrays."""
    t = np.arange(wl.nq, dtype=np.int64)
    if wl.layout == "decode":
        assert wl.n_seq == wl.nq
        seq = t
        pos = np.full(wl.nq, wl.l_max - 1, dtype=np.int64)
    elif wl.layout == "tail":
        seq = np.zeros(wl.nq, dtype=np.int64)
        pos = wl.l_max - wl.nq + t
    elif wl.layout == "prefill":
        assert wl.nq <= wl.l_max
        seq = np.zeros(wl.nq, dtype=np.int64)
        pos = t
    else:
        raise ValueError(wl.layout)
    return seq.astype(np.int32), pos.astype(np.int32)


def _rng(seed: int, wl: Workload, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, wl.wid, *key]))


def queries(wl: Workload, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """q [nq, H, d] (uint16 bf16 bits, or float32) and w [nq, H] float32."""
    g = _rng(seed, wl, _TAG_QUERY)
    q32 = g.standard_normal((wl.nq, wl.n_heads, wl.head_dim), dtype=np.float32)
    w = (g.standard_normal((wl.nq, wl.n_heads), dtype=np.float32) * np.float32(wl.w_scale))
    w = w.astype(np.float32)
    if wl.dtype == BF16:
        return f32_to_bf16_bits(q32), w
    return q32, w


def _q_as_f32(wl: Workload, q: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(q) if wl.dtype == BF16 else q


def _positive_heads(w_t: np.ndarray) -> np.ndarray:
    pos = np.nonzero(w_t > 0)[0]
    return pos if pos.size else np.arange(w_t.size)


def _plants(wl: Workload, seed: int, seq: int, w: np.ndarray,
            q_seq: np.ndarray, q_pos: np.ndarray) -> List[Tuple[int, int, int]]:
    """Planted keys of one sequence as (key position u, query t, head j) triples."""
    g = _rng(seed, wl, _TAG_PLANT, seq)
    out: List[Tuple[int, int, int]] = []
    if wl.plant == "points":
        # n_plant keys, each aimed at a random query (on this sequence) and head,
        # at a random position inside that query's causal prefix; no position twice.
        ts = np.nonzero(q_seq == seq)[0]
        used = set()
        tries = 0
        while len(out) < wl.n_plant and tries < 100 * max(1, wl.n_plant):
            tries += 1
            t = int(ts[g.integers(ts.size)])
            j = int(g.integers(wl.n_heads))
            u = int(g.integers(int(q_pos[t]) + 1))
            if u in used:
                continue
            used.add(u)
            out.append((u, t, j))
    elif wl.plant == "fraction":
        # 1% of the sequence's keys aimed at its own query along positive-weight heads
        t = int(np.nonzero(q_seq == seq)[0][0])
        n = int(round(0.01 * (int(q_pos[t]) + 1)))
        us = g.choice(int(q_pos[t]) + 1, size=n, replace=False)
        heads = _positive_heads(w[t])
        js = heads[g.integers(heads.size, size=n)]
        out = [(int(u), t, int(j)) for u, j in zip(us, js)]
    elif wl.plant == "hot_heads":
        # MISA recipe: 8 "hot" heads per query (positive weight first); n_plant blocks,
        # each with half of its keys planted along one hot head.
        t = int(np.nonzero(q_seq == seq)[0][0])
        B = wl.block
        n_blocks = (int(q_pos[t]) + 1) // B
        order = np.argsort(-w[t], kind="stable")
        pos_first = [int(j) for j in order if w[t, j] > 0]
        rest = [int(j) for j in order if w[t, j] <= 0]
        cand = np.array(pos_first + rest)
        n_hot = min(max(wl.n_active_heads, 1), wl.n_heads)
        hot = g.permutation(cand[:max(n_hot, min(len(pos_first), 2 * n_hot))])[:n_hot]
        blocks = g.choice(n_blocks, size=min(wl.n_plant, n_blocks), replace=False)
        for b in blocks:
            j = int(hot[g.integers(hot.size)])
            us = b * B + g.choice(B, size=B // 2, replace=False)
            out.extend((int(u), t, j) for u in us)
    elif wl.plant == "blocks":
        # HISA recipe: n_plant "relevant" blocks per query; in each a fraction
        # rho ~ U(0.1, 0.6) of its keys planted along positive-weight heads.
        t = int(np.nonzero(q_seq == seq)[0][0])
        B = wl.block
        n_blocks = (int(q_pos[t]) + 1) // B
        heads = _positive_heads(w[t])
        blocks = g.choice(n_blocks, size=min(wl.n_plant, n_blocks), replace=False)
        for b in blocks:
            rho = g.uniform(0.1, 0.6)
            n = int(round(rho * B))
            us = b * B + g.choice(B, size=n, replace=False)
            js = heads[g.integers(heads.size, size=n)]
            out.extend((int(u), t, int(j)) for u, j in zip(us, js))
    else:
        raise ValueError(wl.plant)
    return out


def keys(wl: Workload, seq: int, q: np.ndarray, w: np.ndarray, seed: int = 0,
         l_max: Optional[int] = None) -> np.ndarray:
    """Key cache of one sequence: [l_max, d] uint16 bf16 bits (or float32).

    Keys are drawn N(0, 1) in independently seeded chunks of KEY_CHUNK rows; the
    planted rows are then overwritten with ``q[t, j] + 0.3 * noise``.
    """
    L = wl.l_max if l_max is None else l_max
    d = wl.head_dim
    k32 = np.empty((L, d), dtype=np.float32)
    for c in range((L + KEY_CHUNK - 1) // KEY_CHUNK):
        lo, hi = c * KEY_CHUNK, min(L, (c + 1) * KEY_CHUNK)
        g = _rng(seed, wl, _TAG_KEYS, seq, c)
        k32[lo:hi] = g.standard_normal((hi - lo, d), dtype=np.float32)
    q_seq, q_pos = positions(wl)
    plants = _plants(wl, seed, seq, w, q_seq, q_pos)
    if plants:
        qf = _q_as_f32(wl, q)
        g = _rng(seed, wl, _TAG_PLANT, seq, 1)
        noise = g.standard_normal((len(plants), d), dtype=np.float32)
        for i, (u, t, j) in enumerate(plants):
            if u < L:
                k32[u] = qf[t, j] + np.float32(0.3) * noise[i]
    if wl.dtype == BF16:
        return f32_to_bf16_bits(k32)
    return k32


def all_keys(wl: Workload, q: np.ndarray, w: np.ndarray, seed: int = 0,
             threads: int = 8) -> np.ndarray:
    """[n_seq, l_max, d] key caches (threads over sequences; same bytes as one by one)."""
    dt = np.uint16 if wl.dtype == BF16 else np.float32
    out = np.empty((wl.n_seq, wl.l_max, wl.head_dim), dtype=dt)

    def one(s: int) -> None:
        out[s] = keys(wl, s, q, w, seed)

    if threads <= 1 or wl.n_seq == 1:
        for s in range(wl.n_seq):
            one(s)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(wl.n_seq)))
    return out


def make(wl: Workload, seed: int = 0, threads: int = 8) -> Dict[str, np.ndarray]:
    """All inputs of a workload that fits comfortably in host memory."""
    q, w = queries(wl, seed)
    q_seq, q_pos = positions(wl)
    K = all_keys(wl, q, w, seed, threads)
    return {"q": q, "w": w, "k": K, "q_seq": q_seq, "q_pos": q_pos}


def small(wid: int, **kw) -> Workload:
    """A reduced version of workload ``wid`` for parity tests (same recipe)."""
    return WORKLOADS[wid].replace(**kw)
