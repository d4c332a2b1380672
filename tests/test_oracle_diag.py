"""Pins of the diagnostics oracle (oracle/diag.py): brute force on a tiny
case, closed forms (zero queries, two-level logits, one block), the row-sum
invariant, agreement with the attention oracle through the sparse LSE,
nesting of block sizes, optimality of the oracle top-k, and the error
sums."""
import math

import numpy as np
import pytest

from oracle import attn as oat
from oracle import diag as odg
from synth import bf16_bits_to_f64, make_qkv


def _head(T, Hg, Wg, d, seed=0):
    q, k, v = make_qkv(T, Hg, Wg, 1, d, seed)
    return tuple(bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))


def test_brute_force_tiny():
    """Pure-Python loops: every probability from math.exp, sums by hand."""
    rng = np.random.default_rng(0)
    Nq, Nk, d, qb, kvb = 5, 7, 3, 2, 3
    q, k = rng.normal(size=(Nq, d)), rng.normal(size=(Nk, d))
    sc = 0.7
    A = odg.block_mass(q, k, qb, kvb, scale=sc)
    assert A.shape == (3, 3)
    for i in range(3):
        rows = [n for n in range(Nq) if n // qb == i]
        for j in range(3):
            tot = 0.0
            for n in rows:
                z = sum(math.exp(sc * sum(q[n, c] * k[t, c] for c in range(d))) for t in range(Nk))
                tot += sum(math.exp(sc * sum(q[n, c] * k[t, c] for c in range(d)))
                           for t in range(Nk) if t // kvb == j) / z
            assert A[i, j] == pytest.approx(tot / len(rows), rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("Nq,Nk,kvb", [(300, 257, 4), (128, 1000, 7), (129, 64, 64), (50, 33, 1)])
def test_rows_sum_to_one(Nq, Nk, kvb):
    rng = np.random.default_rng(Nq + Nk)
    q, k = rng.normal(size=(Nq, 16)) * 2, rng.normal(size=(Nk, 16)) * 2
    A = odg.block_mass(q, k, 128, kvb)
    np.testing.assert_allclose(A.sum(axis=1), 1.0, rtol=1e-12)
    assert (A >= 0).all()


def test_zero_queries_give_block_sizes():
    Nk, kvb = 130, 4
    A = odg.block_mass(np.zeros((200, 8)), np.random.default_rng(1).normal(size=(Nk, 8)), 128, kvb)
    sizes = np.array([4] * 32 + [2]) / Nk
    np.testing.assert_allclose(A, np.tile(sizes, (2, 1)), rtol=1e-14)


def test_two_level_closed_form():
    """Keys of block 0 give logit a, every other key logit 0."""
    d, Nk, kvb, a = 4, 40, 8, 1.3
    k = np.zeros((Nk, d))
    k[:kvb, 0] = 1.0
    q = np.zeros((3, d))
    q[:, 0] = a                      # scale 1: logit a on block 0
    A = odg.block_mass(q, k, 128, kvb, scale=1.0)
    m0 = kvb * math.exp(a) / (kvb * math.exp(a) + (Nk - kvb))
    assert A[0, 0] == pytest.approx(m0, rel=1e-14)
    np.testing.assert_allclose(A[0, 1:], (1 - m0) / 4, rtol=1e-13)


def test_one_block_holds_everything():
    q, k, _ = _head(1, 4, 20, 32, seed=3)
    A = odg.block_mass(q, k, 128, 4096)
    np.testing.assert_allclose(A, 1.0, rtol=1e-13)


def test_sparse_lse_identity():
    """With one query per block and no shift, the sparse attention's LSE is
    the dense LSE plus ln of the retained mass of its list."""
    q, k, v = _head(1, 6, 20, 32, seed=5)
    N = q.shape[0]
    kvb, M = 4, N // 4
    rng = np.random.default_rng(6)
    idx = np.stack([np.sort(rng.choice(M, 9, replace=False)) for _ in range(N)])
    cnt = np.full(N, 9)
    _, lse_s = oat.attn_fwd(q, k, v, 1, kvb, idx, None, cnt)
    _, lse_d = oat.dense_attn(q, k, v)
    A = odg.block_mass(q, k, 1, kvb, lse=lse_d)
    cov = odg.plan_coverage(A, idx, cnt)
    np.testing.assert_allclose(np.log(cov), lse_s - lse_d, rtol=0, atol=1e-12)
    # the attention oracle's LSE as input equals the internal normaliser
    np.testing.assert_allclose(A, odg.block_mass(q, k, 1, kvb), rtol=1e-12)


def test_nested_block_sizes():
    """Masses at 8-token blocks are pairwise sums of the 4-token ones, so an
    oracle top-2s at 4 tokens retains at least the top-s at 8 tokens."""
    q, k, _ = _head(2, 8, 16, 64, seed=8)
    A4 = odg.block_mass(q, k, 128, 4)
    A8 = odg.block_mass(q, k, 128, 8)
    np.testing.assert_allclose(A8, A4.reshape(A4.shape[0], -1, 2).sum(axis=2), rtol=1e-12)
    for s in (4, 16, 40):
        i4, c4 = odg.oracle_topk(A4, 2 * s)
        i8, c8 = odg.oracle_topk(A8, s)
        r4, r8 = odg.plan_coverage(A4, i4, c4), odg.plan_coverage(A8, i8, c8)
        assert (r4 >= r8 - 1e-12).all()


def test_oracle_topk_is_optimal_and_ordered():
    rng = np.random.default_rng(9)
    A = rng.gamma(0.3, size=(4, 60))
    A[0, 10] = A[0, 11] = A[0].max() + 1.0          # tie -> lower index first
    idx, cnt = odg.oracle_topk(A, 7)
    assert (cnt == 7).all() and (np.diff(idx, axis=1) > 0).all()
    cov = odg.plan_coverage(A, idx, cnt)
    np.testing.assert_allclose(cov, np.sort(A, axis=1)[:, -7:].sum(axis=1), rtol=1e-14)
    for _ in range(50):
        other = np.stack([rng.choice(60, 7, replace=False) for _ in range(4)])
        assert (odg.plan_coverage(A, other, cnt) <= cov + 1e-14).all()
    i1, _ = odg.oracle_topk(A[:1, :12], 1)
    assert i1[0, 0] == 10


def test_coverage_skips_invalid_and_counts_order():
    A = np.array([[0.5, 0.25, 0.125, 0.125]])
    idx = np.array([[2, -1, 7, 0, 1]])
    assert odg.plan_coverage(A, idx, np.array([4]))[0] == 0.625
    assert odg.plan_coverage(A, idx, np.array([0]))[0] == 0.0
    assert odg.plan_coverage(A, idx, np.array([9]))[0] == 0.875   # count clamped to the row


def test_output_error_sums():
    O = np.array([[1.0, 2.0], [3.0, -1.0]])
    num, den = odg.output_error(O + np.array([[0.5, 0], [0, -1.0]]), O)
    assert (num, den) == (1.25, 15.0)
    assert odg.relative_error(2 * O, O) == pytest.approx(1.0, rel=1e-15)
    assert odg.relative_error(O, O) == 0.0
