"""Pins of the sparse-attention oracle against things other than itself.

Closed forms (one selected row, identical keys, zero query), a library
routine on the gathered rows (PyTorch's scaled_dot_product_attention, CPU,
float64), invariances of the index list (padding, order), and the
independent pure-Python brute force on tiny inputs.
"""
import numpy as np
import torch

from oracle import attention as A
from oracle import brute


def _inputs(rng, H, D, L):
    return rng.standard_normal((H, D)), rng.standard_normal((L, D))


def test_one_selected_row_gives_its_value():
    rng = np.random.default_rng(1)
    q, C = _inputs(rng, 5, 12, 30)
    for u in (0, 7, 29):
        o, mag = A.sparse_mla_row(q, C, np.array([u, -1, 30, -5]), 8, 0.3)
        assert np.array_equal(o, np.broadcast_to(C[u, :8], o.shape))
        assert np.array_equal(mag, np.abs(o))


def test_identical_keys_and_zero_query_give_the_mean():
    rng = np.random.default_rng(2)
    q, C = _inputs(rng, 4, 10, 40)
    idx = rng.choice(40, size=17, replace=False)
    # q = 0: every score is 0, so the weights are uniform
    o, _ = A.sparse_mla_row(np.zeros_like(q), C, idx, 6, 0.5)
    assert np.allclose(o, C[idx, :6].mean(axis=0), rtol=0, atol=1e-14)
    # equal keys along the scored dimensions, different values: uniform again
    C2 = C.copy()
    C2[:, 6:] = C2[0, 6:]
    q2 = q.copy()
    q2[:, :6] = 0.0
    o2, _ = A.sparse_mla_row(q2, C2, idx, 6, 1.7)
    assert np.allclose(o2, C2[idx, :6].mean(axis=0), rtol=0, atol=1e-14)


def test_matches_library_attention_on_the_gathered_rows():
    rng = np.random.default_rng(3)
    for _ in range(10):
        H, D, L = int(rng.integers(1, 9)), int(rng.integers(2, 40)), int(rng.integers(1, 200))
        d_v = int(rng.integers(1, D + 1))
        q, C = _inputs(rng, H, D, L)
        k = int(rng.integers(1, L + 1))
        idx = rng.choice(L, size=k, replace=False)
        scale = float(rng.uniform(0.05, 1.0))
        o, _ = A.sparse_mla_row(q, C, idx, d_v, scale)
        G = torch.from_numpy(C[idx])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], G[None, None], G[None, None, :, :d_v], scale=scale)
        assert np.allclose(o, ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_padding_and_order_do_not_matter():
    rng = np.random.default_rng(4)
    q, C = _inputs(rng, 6, 16, 64)
    idx = rng.choice(64, size=20, replace=False)
    o, _ = A.sparse_mla_row(q, C, idx, 16, 0.25)
    padded = np.concatenate([idx[:7], [-1, 64, 1000], idx[7:], [-1] * 5])
    op, _ = A.sparse_mla_row(q, C, padded, 16, 0.25)
    assert np.allclose(o, op, rtol=0, atol=1e-14)
    orr, _ = A.sparse_mla_row(q, C, idx[rng.permutation(20)], 16, 0.25)
    assert np.allclose(o, orr, rtol=0, atol=1e-14)
    z, zm = A.sparse_mla_row(q, C, np.array([-1, -1, 64]), 16, 0.25)
    assert not z.any() and not zm.any()


def test_matches_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(30):
        H, D, L = int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 30))
        d_v = int(rng.integers(1, D + 1))
        q, C = _inputs(rng, H, D, L)
        idx = rng.integers(-2, L + 2, size=int(rng.integers(1, 12)))   # repeats and padding
        scale = float(rng.uniform(0.1, 2.0))
        o, _ = A.sparse_mla_row(q, C, idx, d_v, scale)
        b = np.array(brute.sparse_mla(q.tolist(), C.tolist(), idx.tolist(), d_v, scale))
        assert np.allclose(o, b, rtol=1e-12, atol=1e-12)
