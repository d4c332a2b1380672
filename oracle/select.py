"""IBCS selector oracle: KV-block mean pooling, intra-query-block k-means,
and block scores.

Test infrastructure only (see ``oracle/__init__``).

Follows the AB-Attention page (onedev.kr/papers/1521), section "무엇과 다른가"
(the Intra-Block Clustering Selector):

* queries are cut into blocks of the execution-tile height (128), keys and
  values into much smaller blocks (4 tokens);
* inside each query block only, one k-means iteration forms 8 query clusters,
  giving each cluster a centroid and a share of the block's queries;
* a KV block's score is the share-weighted average, over the clusters, of the
  softmax mass that the centroid puts on that block's pooled key.

Readings where the page is silent:

* pooled key = mean of the block's keys (the last block averages its valid
  rows only);
* k-means starts from contiguous segment means (segment c = rows
  [floor(c n / C), floor((c + 1) n / C))), the position-based 16-query means
  that the ablation paragraph of "전제와 한계" names; one iteration = one
  assignment by squared Euclidean distance (ties to the lowest cluster) and
  one update; a cluster left empty keeps its centroid with share 0; a
  cluster whose starting segment is empty is inactive (share 0, centroid 0);
* the softmax runs over all M KV blocks of the head with scale 1/sqrt(d).

The k-means is a chain of discrete decisions, so it is evaluated in fp32 in
this exact operation order (the HIP kernel uses the same one): member sums
run over rows in ascending order with one rounding per add; a mean is that
sum divided by the member count with one IEEE division; a distance is
sum over dims 0..d-1, ascending, of (q_k - mu_k)^2 with a rounded subtract,
a rounded multiply and a rounded add (no fused multiply-add).  Scores are
then computed in fp64 from those fp32 centroids.
"""
from __future__ import annotations

import numpy as np


def pool_keys(k: np.ndarray, kv_block: int) -> np.ndarray:
    """k: (N, d) fp64 -> (M, d) fp64 pooled keys, M = ceil(N / kv_block)."""
    N, d = k.shape
    M = -(-N // kv_block)
    out = np.empty((M, d), dtype=np.float64)
    full = N // kv_block
    if full:
        out[:full] = k[: full * kv_block].reshape(full, kv_block, d).mean(axis=1)
    if M > full:
        out[full] = k[full * kv_block:].mean(axis=0)
    return out


def _member_means(q: np.ndarray, assign: np.ndarray, C: int, prev: np.ndarray):
    """fp32 means of the rows assigned to each cluster (ascending row order).

    q: (nb, n, d) fp32, assign: (nb, n) int.  Clusters without members keep
    ``prev``.  Returns (mu (nb, C, d) fp32, counts (nb, C) int64).
    """
    nb, n, d = q.shape
    acc = np.zeros((nb, C, d), dtype=np.float32)
    counts = np.zeros((nb, C), dtype=np.int64)
    bi = np.arange(nb)
    for r in range(n):
        a = assign[:, r]
        acc[bi, a] = acc[bi, a] + q[:, r]
        counts[bi, a] += 1
    mu = prev.copy()
    has = counts > 0
    denom = counts.astype(np.float32)
    mu[has] = acc[has] / denom[has][:, None]
    return mu, counts


def kmeans_blocks(q: np.ndarray, C: int, iters: int):
    """k-means inside each of ``nb`` query blocks of equal size ``n``.

    q: (nb, n, d) fp32 (bf16 values).  Returns
    (mu (nb, C, d) fp32, w (nb, C) fp32, assign (nb, n) int64).
    """
    nb, n, d = q.shape
    seg = np.array([(c * n) // C for c in range(C + 1)])
    active = seg[1:] > seg[:-1]                      # clusters with a starting segment
    row_seg = np.searchsorted(seg[1:], np.arange(n), side="right")
    assign = np.broadcast_to(row_seg, (nb, n)).copy()
    mu, counts = _member_means(q, assign, C, np.zeros((nb, C, d), np.float32))
    for _ in range(iters):
        dist = np.zeros((nb, n, C), dtype=np.float32)
        for kk in range(d):
            diff = q[:, :, kk][:, :, None] - mu[:, :, kk][:, None, :]
            dist = dist + diff * diff
        dist[:, :, ~active] = np.inf
        assign = np.argmin(dist, axis=2)             # first minimum = lowest cluster
        mu, counts = _member_means(q, assign, C, mu)
    w = counts.astype(np.float32) / np.float32(n)
    return mu, w, assign


def kmeans_head(q32: np.ndarray, q_block: int, C: int, iters: int):
    """All query blocks of one head.  q32: (N, d) fp32 -> (mu, w) per block."""
    N, d = q32.shape
    nqb = -(-N // q_block)
    full = N // q_block
    mu = np.zeros((nqb, C, d), np.float32)
    w = np.zeros((nqb, C), np.float32)
    if full:
        m, ww, _ = kmeans_blocks(q32[: full * q_block].reshape(full, q_block, d), C, iters)
        mu[:full], w[:full] = m, ww
    if nqb > full:
        m, ww, _ = kmeans_blocks(q32[full * q_block:][None], C, iters)
        mu[full], w[full] = m[0], ww[0]
    return mu, w


def scores_from_centroids(mu: np.ndarray, w: np.ndarray, kbar: np.ndarray,
                          chunk: int = 32) -> np.ndarray:
    """S (nqb, M) fp64: S_ij = sum_c w_ic softmax_j(mu_ic . kbar_j / sqrt(d))."""
    nqb, C, d = mu.shape
    M = kbar.shape[0]
    S = np.empty((nqb, M), dtype=np.float64)
    kT = np.ascontiguousarray(kbar.T)
    inv = 1.0 / np.sqrt(d)
    for i0 in range(0, nqb, chunk):
        i1 = min(nqb, i0 + chunk)
        logits = (mu[i0:i1].astype(np.float64).reshape(-1, d) @ kT) * inv
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        p = p.reshape(i1 - i0, C, M)
        S[i0:i1] = np.einsum("bc,bcm->bm", w[i0:i1].astype(np.float64), p)
    return S


def select_scores_head(q_bits: np.ndarray, k_bits: np.ndarray, q_block: int,
                       kv_block: int, C: int, iters: int):
    """One head: bf16 bit arrays (N, d) -> (S fp64 (nqb, M), mu fp32, w fp32)."""
    from synth import bf16_bits_to_f32, bf16_bits_to_f64
    q32 = bf16_bits_to_f32(q_bits)
    k64 = bf16_bits_to_f64(k_bits)
    mu, w = kmeans_head(q32, q_block, C, iters)
    kbar = pool_keys(k64, kv_block)
    return scores_from_centroids(mu, w, kbar), mu, w
