"""Seeded synthetic inputs for the sparse-attention consumer of the index list.

This module only draws inputs: the attention queries, the latent cache rows,
the per-query (sequence, position) pairs and the index lists.  It contains
none of the attention arithmetic, so both the CPU oracle and the GPU path may
be fed from it.

Shapes follow absorbed multi-head latent attention (the Sparse MLA operator
the HISA review names as the consumer of the selected indices): every token
has one latent row of d_qk = 512 + 64 values (compressed key-value part plus
a rotary part) that all attention heads share as the key, and whose first
d_v = 512 values are the value; 128 attention heads; the index list of each
query holds top_k = 2048 distinct positions of its prefix, the indexer's
output size.  Values are N(0, 1) rounded to bf16.  Each cache row is seeded
by (seed, sequence, position) alone, so any set of rows regenerates to the
same bytes without generating the rest of the cache; the index lists are
uniform draws without replacement from the prefix (real lists cluster, which
only helps a gather).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

from . import f32_to_bf16_bits

_NS = 6            # seed namespace, distinct from the indexer workloads
_TAG_QUERY = 0
_TAG_ROW = 1
_TAG_IDX = 2


@dataclasses.dataclass(frozen=True)
class MlaWorkload:
    name: str
    nq: int
    n_seq: int
    l_max: int
    n_heads: int = 128
    d_qk: int = 576
    d_v: int = 512
    top_k: int = 2048
    layout: str = "decode"   # decode: query t on its own cache at l_max - 1;
                             # tail: one cache, queries at the last nq positions
    scale: float = 1.0 / 192 ** 0.5   # softmax scale of a 128 + 64 q/k head

    def replace(self, **kw) -> "MlaWorkload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, MlaWorkload] = {
    "sparse_mla_decode_L128K_H128": MlaWorkload("sparse_mla_decode_L128K_H128", nq=64, n_seq=64,
                                                l_max=131072),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _NS, *key]))


def positions(wl: MlaWorkload) -> Tuple[np.ndarray, np.ndarray]:
    t = np.arange(wl.nq, dtype=np.int64)
    if wl.layout == "decode":
        assert wl.n_seq == wl.nq
        seq, pos = t, np.full(wl.nq, wl.l_max - 1, dtype=np.int64)
    elif wl.layout == "tail":
        assert wl.nq <= wl.l_max
        seq, pos = np.zeros(wl.nq, dtype=np.int64), wl.l_max - wl.nq + t
    else:
        raise ValueError(wl.layout)
    return seq.astype(np.int32), pos.astype(np.int32)


def queries(wl: MlaWorkload, seed: int = 0) -> np.ndarray:
    """q [nq, n_heads, d_qk] as bf16 bits."""
    g = _rng(seed, _TAG_QUERY)
    return f32_to_bf16_bits(g.standard_normal((wl.nq, wl.n_heads, wl.d_qk), dtype=np.float32))


def rows(wl: MlaWorkload, seq: int, pos: np.ndarray, seed: int = 0) -> np.ndarray:
    """The latent rows of one sequence at the given positions, [n, d_qk] bf16 bits."""
    pos = np.asarray(pos, dtype=np.int64).reshape(-1)
    out = np.empty((pos.size, wl.d_qk), dtype=np.uint16)
    for n, p in enumerate(pos):
        out[n] = f32_to_bf16_bits(_rng(seed, _TAG_ROW, seq, int(p)).standard_normal(
            wl.d_qk, dtype=np.float32))
    return out


def cache(wl: MlaWorkload, seed: int = 0) -> np.ndarray:
    """The whole cache [n_seq, l_max, d_qk] (bf16 bits); small workloads only."""
    return np.stack([rows(wl, s, np.arange(wl.l_max), seed) for s in range(wl.n_seq)])


def index_lists(wl: MlaWorkload, seed: int = 0) -> np.ndarray:
    """idx [nq, top_k] int32: top_k distinct positions of each query's prefix in
    random order, or the whole (shuffled) prefix padded with -1 when shorter."""
    _, pos = positions(wl)
    out = np.full((wl.nq, wl.top_k), -1, dtype=np.int32)
    for t in range(wl.nq):
        n = int(pos[t]) + 1
        g = _rng(seed, _TAG_IDX, t)
        if n <= wl.top_k:
            out[t, :n] = g.permutation(n)
        else:
            out[t] = g.choice(n, size=wl.top_k, replace=False)
    return out
