"""Pins of the selector oracle (pooling, k-means, block scores) against
special cases, brute force and an independent library (torch, fp64, CPU)."""
import numpy as np
import pytest
import torch

from oracle import select as osel
from synth import bf16_bits_to_f32, bf16_bits_to_f64, f64_to_bf16_bits, make_qkv


def _bf16(x):
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def test_pool_identity_for_unit_blocks():
    rng = np.random.default_rng(0)
    k = _bf16(rng.standard_normal((37, 16)))
    assert np.array_equal(osel.pool_keys(k, 1), k)


@pytest.mark.parametrize("N,b", [(64, 4), (66, 4), (130, 64), (5, 8)])
def test_pool_brute_force(N, b):
    rng = np.random.default_rng(N + b)
    k = _bf16(rng.standard_normal((N, 8)))
    got = osel.pool_keys(k, b)
    M = -(-N // b)
    assert got.shape == (M, 8)
    for j in range(M):
        rows = range(j * b, min(N, (j + 1) * b))
        want = [sum(float(k[r, c]) for r in rows) / len(rows) for c in range(8)]
        np.testing.assert_allclose(got[j], want, rtol=1e-15, atol=1e-15)


def test_kmeans_single_cluster_is_block_mean():
    rng = np.random.default_rng(1)
    q = bf16_bits_to_f32(f64_to_bf16_bits(rng.standard_normal((3, 128, 32))))
    mu, w, assign = osel.kmeans_blocks(q, 1, 1)
    np.testing.assert_allclose(mu[:, 0], q.astype(np.float64).mean(axis=1), rtol=0, atol=2e-6)
    assert np.all(w == 1.0) and np.all(assign == 0)


@pytest.mark.parametrize("n,C", [(128, 8), (120, 8), (80, 8), (16, 8), (5, 8)])
def test_kmeans_zero_iterations_are_segment_means(n, C):
    """iters = 0 gives the position-based segment means of the ablation
    (16-query segments for a full 128-query block and 8 clusters)."""
    rng = np.random.default_rng(n)
    q = bf16_bits_to_f32(f64_to_bf16_bits(rng.standard_normal((2, n, 16))))
    mu, w, _ = osel.kmeans_blocks(q, C, 0)
    for c in range(C):
        lo, hi = (c * n) // C, ((c + 1) * n) // C
        if hi > lo:
            np.testing.assert_allclose(mu[:, c], q[:, lo:hi].astype(np.float64).mean(axis=1),
                                       atol=2e-6)
            assert np.all(w[:, c] == np.float32(hi - lo) / np.float32(n))
        else:
            assert np.all(w[:, c] == 0) and np.all(mu[:, c] == 0)
    if n == 128:
        assert np.all(w == np.float32(16 / 128))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)


def _kmeans_fp64_reference(qb, C, iters):
    """Textbook k-means in fp64 from the segment-mean start, written plainly."""
    n = len(qb)
    seg = [(c * n) // C for c in range(C + 1)]
    active = [seg[c + 1] > seg[c] for c in range(C)]
    mu = [qb[seg[c]:seg[c + 1]].mean(axis=0) if active[c] else np.zeros(qb.shape[1])
          for c in range(C)]
    assign = [next(c for c in range(C) if seg[c] <= r < seg[c + 1]) for r in range(n)]
    for _ in range(iters):
        assign = []
        for r in range(n):
            best, bd = None, None
            for c in range(C):
                if not active[c]:
                    continue
                dd = float(((qb[r] - mu[c]) ** 2).sum())
                if bd is None or dd < bd:
                    best, bd = c, dd
            assign.append(best)
        for c in range(C):
            mem = [r for r in range(n) if assign[r] == c]
            if mem:
                mu[c] = qb[mem].mean(axis=0)
    w = [sum(1 for a in assign if a == c) / n for c in range(C)]
    return np.array(mu), np.array(w), np.array(assign)


@pytest.mark.parametrize("seed", range(4))
def test_kmeans_matches_textbook_fp64_on_separated_data(seed):
    """Clustered queries (clear margins): the fp32 ordered k-means reaches the
    same assignment as a plain fp64 k-means, centroids within fp32 rounding."""
    rng = np.random.default_rng(seed)
    n, C, d = 48, 4, 16
    centers = rng.standard_normal((6, d)) * 4
    lab = rng.integers(0, 6, size=n)
    x = centers[lab] + 0.1 * rng.standard_normal((n, d))
    q32 = bf16_bits_to_f32(f64_to_bf16_bits(x))
    mu, w, assign = osel.kmeans_blocks(q32[None], C, 1)
    rmu, rw, rassign = _kmeans_fp64_reference(q32.astype(np.float64), C, 1)
    assert np.array_equal(assign[0], rassign)
    np.testing.assert_allclose(mu[0], rmu, atol=1e-5)
    np.testing.assert_allclose(w[0], rw, atol=1e-7)


def test_kmeans_brute_force_invariants():
    """Every row sits at an argmin of its distance to the starting centroids
    (ties to the lowest), and every updated centroid is its members' mean."""
    rng = np.random.default_rng(11)
    q = bf16_bits_to_f32(f64_to_bf16_bits(rng.standard_normal((4, 40, 8))))
    C = 8
    mu, w, assign = osel.kmeans_blocks(q, C, 1)
    mu0, _, _ = osel.kmeans_blocks(q, C, 0)
    for b in range(4):
        for r in range(40):
            dd = ((q[b, r].astype(np.float64) - mu0[b].astype(np.float64)) ** 2).sum(axis=1)
            assert dd[assign[b, r]] <= dd.min() * (1 + 1e-6) + 1e-12
        for c in range(C):
            mem = assign[b] == c
            if mem.any():
                np.testing.assert_allclose(mu[b, c], q[b, mem].astype(np.float64).mean(axis=0),
                                           atol=2e-6)
                assert w[b, c] == np.float32(mem.sum()) / np.float32(40)
        assert abs(float(w[b].sum()) - 1.0) < 1e-6


def test_kmeans_tie_goes_to_lowest_cluster():
    a = np.zeros(4, np.float32); a[0] = 1.0
    b = np.zeros(4, np.float32); b[1] = 1.0
    q = np.stack([a, b, a, b])[None]           # both segments have the same mean
    mu, w, assign = osel.kmeans_blocks(q, 2, 1)
    assert np.all(assign == 0)
    assert w[0, 0] == 1.0 and w[0, 1] == 0.0
    np.testing.assert_array_equal(mu[0, 0], (a + b) / 2)


def test_scores_unit_blocks_equal_softmax_attention_probabilities():
    """q_block = kv_block = 1 and one cluster: S_ij is the softmax attention
    probability of query i on key j (torch fp64 as the independent reference)."""
    qb, kb, _ = make_qkv(1, 6, 7, 1, 32, seed=3)
    S, mu, w = osel.select_scores_head(qb[0, 0], kb[0, 0], 1, 1, 1, 1)
    q = torch.from_numpy(bf16_bits_to_f64(qb[0, 0]))
    k = torch.from_numpy(bf16_bits_to_f64(kb[0, 0]))
    ref = torch.softmax(q @ k.T / np.sqrt(32.0), dim=-1).numpy()
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-300)


def test_scores_two_clusters_weighted_mixture():
    """Two distinct query rows repeated in two segments: S is the 0.5/0.5
    mixture of the two rows' softmax distributions over the pooled keys."""
    rng = np.random.default_rng(5)
    d = 16
    a = _bf16(rng.standard_normal(d))
    b = _bf16(rng.standard_normal(d))
    qrows = np.stack([a, a, b, b])
    k = _bf16(rng.standard_normal((24, d)))
    S, mu, w = osel.select_scores_head(f64_to_bf16_bits(qrows), f64_to_bf16_bits(k), 4, 4, 2, 1)
    kbar = torch.from_numpy(k).reshape(6, 4, d).mean(dim=1)
    pa = torch.softmax(torch.from_numpy(a) @ kbar.T / 4.0, dim=-1)
    pb = torch.softmax(torch.from_numpy(b) @ kbar.T / 4.0, dim=-1)
    np.testing.assert_allclose(S[0], (0.5 * pa + 0.5 * pb).numpy(), rtol=1e-12)


def test_scores_are_distributions():
    qb, kb, _ = make_qkv(2, 8, 16, 1, 64, seed=4)
    S, mu, w = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, 4, 8, 1)
    assert S.shape == (2, 64)
    assert np.all(S > 0)
    np.testing.assert_allclose(S.sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
