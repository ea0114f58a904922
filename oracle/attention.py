"""Plain float64 NumPy oracle of the sparse-attention consumer of the index list.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports this module.

Sources (page titles as printed; sections as they appear on each page):

* "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse Attention"
  (paper review), key terms and section 3: the selected token indices are the
  input of a downstream Sparse MLA operator, which HISA leaves unchanged.
* "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse"
  (review), section 1: with the indexer's top-k tokens per query, the core
  attention costs O(L k) instead of O(L^2).

The pages give no formula for the operator.  Reading R19 (also listed with the
design notes): per query t and attention head h, ordinary scaled-softmax
attention restricted to the rows the index list names, in the absorbed form of
multi-head latent attention: one latent cache row c[u] of D = d_qk values per
token serves as the key of every head, and its first d_v values are the value.

    s[h, i] = scale * q[t, h] . c[idx[t, i]]
    o[t, h] = sum_i softmax_i(s[h, :]) * c[idx[t, i], :d_v]

over the entries of idx[t] inside [0, prefix length) (others, e.g. the -1
padding of a short prefix, are skipped; a repeated entry counts each time).
A row with no valid entry outputs zeros.

Pins (tests/test_oracle_attention.py): one selected row gives that row's value;
identical keys or q = 0 give the plain mean of the selected values; the result
equals PyTorch's scaled_dot_product_attention on the gathered rows (CPU,
float64); padding and order of the index list do not change it; the
pure-Python brute force in brute.py agrees on tiny inputs.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def valid_entries(idx_t: np.ndarray, n_keys: int) -> np.ndarray:
    """The entries of one index list that name a row of the prefix (R19)."""
    idx_t = np.asarray(idx_t, dtype=np.int64)
    return idx_t[(idx_t >= 0) & (idx_t < n_keys)]


def sparse_mla_row(q_t: np.ndarray, kv_rows: np.ndarray, idx_t: np.ndarray, d_v: int,
                   scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one query's heads over its selected latent rows.

    q_t [H, D] and kv_rows [n_keys, D] are float64 (the query's prefix of its
    cache, already widened from bf16); idx_t [k] holds row ids.  Returns
    o [H, d_v] and mag [H, d_v] = sum_i p[h, i] * |v_i|, the scale the
    matching tolerance is taken relative to."""
    sel = valid_entries(idx_t, kv_rows.shape[0])
    H = q_t.shape[0]
    if sel.size == 0:
        z = np.zeros((H, d_v))
        return z, z.copy()
    C = kv_rows[sel]                       # [n, D] the gathered rows
    V = C[:, :d_v]
    s = scale * (q_t @ C.T)                # [H, n]
    s = s - s.max(axis=1, keepdims=True)   # softmax is shift-invariant per row
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V, p @ np.abs(V)
