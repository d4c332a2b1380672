"""Pins of the attention backward oracle (oracle/attn.py: attn_bwd):
central finite differences of the forward oracle (shifts, a repeated
block, a partial last block, a ragged query block), torch autograd of fp64
SDPA when every block is listed, zero gradients for unlisted keys, and
invalid entries ignored."""
import numpy as np
import pytest
import torch

from oracle import attn as oat


def _loss(q, k, v, dout, qb, kvb, idx, bias, cnt, scale):
    O, _ = oat.attn_fwd(q, k, v, qb, kvb, idx, bias, cnt, scale=scale)
    return float((dout * O).sum())


def test_finite_differences():
    rng = np.random.default_rng(0)
    Nq, Nk, d, qb, kvb, sc = 6, 10, 3, 4, 3, 0.8
    q, k, v, dout = (rng.normal(size=(n, d)) for n in (Nq, Nk, Nk, Nq))
    idx = np.array([[0, 3, 3, 1], [2, 3, 0, 0]])      # block 3 holds one key; repeats
    bias = rng.normal(size=idx.shape).astype(np.float32)
    cnt = np.array([4, 3])
    dq, dk, dv = oat.attn_bwd(q, k, v, dout, qb, kvb, idx, bias, cnt, scale=sc)
    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dv)):
        for pos in np.ndindex(X.shape):
            x0 = X[pos]
            X[pos] = x0 + h
            lp = _loss(q, k, v, dout, qb, kvb, idx, bias, cnt, sc)
            X[pos] = x0 - h
            lm = _loss(q, k, v, dout, qb, kvb, idx, bias, cnt, sc)
            X[pos] = x0
            assert G[pos] == pytest.approx((lp - lm) / (2 * h), rel=1e-6, abs=1e-8), pos


def test_all_blocks_equal_autograd_of_dense_attention():
    rng = np.random.default_rng(1)
    Nq, Nk, d, kvb = 200, 70, 16, 8
    q, k, v, dout = (rng.normal(size=(n, d)) for n in (Nq, Nk, Nk, Nq))
    M = -(-Nk // kvb)
    idx = np.tile(np.arange(M), (2, 1))
    dq, dk, dv = oat.attn_bwd(q, k, v, dout, 128, kvb, idx, None, np.full(2, M))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    (O * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_unlisted_keys_and_invalid_entries():
    rng = np.random.default_rng(2)
    Nq, Nk, d, kvb = 130, 64, 8, 4
    q, k, v, dout = (rng.normal(size=(n, d)) for n in (Nq, Nk, Nk, Nq))
    idx = np.array([[1, 5, -1, 99, 7], [2, 5, 16, 3, 0]])
    cnt = np.array([5, 3])
    dq, dk, dv = oat.attn_bwd(q, k, v, dout, 128, kvb, idx, None, cnt)
    listed = {1, 5, 7, 2}
    for j in range(Nk // kvb):
        rows = slice(j * kvb, (j + 1) * kvb)
        if j not in listed:
            assert not dk[rows].any() and not dv[rows].any()
    clean = np.array([[1, 5, 7], [2, 5, 16]])
    want = oat.attn_bwd(q, k, v, dout, 128, kvb, clean, None, np.array([3, 2]))
    for a, b in zip((dq, dk, dv), want):
        np.testing.assert_array_equal(a, b)
