"""Seeded synthetic Q/K/V on a video latent grid.

This module is shared by the tests, the benchmark and the oracle.  It holds
no step of the attention method itself: it only draws inputs.  Everything is
deterministic given (grid, heads, head dim, seed).

Recipe (per head h, ``rng = numpy.random.default_rng([seed, h])``, all fp64):

1. ``G`` = d x d standard normal; its QR factor's first 16 rows ``u_m`` are
   orthonormal; they are scaled by sqrt(d / 8).
2. ``Z_Q``, ``Z_K``, ``V``: N x d standard normal each, drawn in that order.
3. Token n <-> (t, y, x) in raster order n = (t * Hg + y) * Wg + x.  Sixteen
   positional features: for pair f = 0..7 the axis is (t, y, x)[f mod 3] and
   the angular rate is (pi / 2) * 2^(-f / 2); feature 2f is the sine and
   2f + 1 the cosine of rate * coordinate.
4. ``P = sum_m phi_m u_m`` (per-channel RMS exactly 1), ``Q = 0.5 Z_Q + P``,
   ``K = 0.5 Z_K + P`` (the same u_m, which makes attention local on the
   grid), ``V = Z_V``.
5. Cast fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even).

The video DiT pages (AB-Attention, BASA) measure on real model activations of
prompt suites that are not available here; these tensors have the same latent
shapes and a tunable locality, nothing more.
"""
from __future__ import annotations

import numpy as np

# Latent grids and heads of the workloads the pages describe.
CONFIGS = {
    # tiny case on a 2x32x32 grid, head dim 64, 64-token KV blocks, top-8
    "tiny_2x32x32": dict(T=2, Hg=32, Wg=32, H=1, d=64, q_block=128, kv_block=64,
                         n_clusters=1, kmeans_iters=1, budget=8, mode="topk"),
    # Wan2.1-1.3B 480p x 81 frames
    "wan13b_480p": dict(T=21, Hg=30, Wg=52, H=12, d=128, q_block=128, kv_block=4,
                        n_clusters=8, kmeans_iters=1, budget=887, mode="sip"),
    # Wan2.1-14B 720p x 81 frames
    "wan14b_720p": dict(T=21, Hg=45, Wg=80, H=40, d=128, q_block=128, kv_block=4,
                        n_clusters=8, kmeans_iters=1, budget=2048, mode="sip"),
    # HunyuanVideo-13B 720p x 129 frames
    "hunyuan_720p": dict(T=33, Hg=45, Wg=80, H=24, d=128, q_block=128, kv_block=4,
                         n_clusters=8, kmeans_iters=1, budget=2272, mode="sip"),
    # BASA-structured 1664x960 x 81 frames (latent 21x60x104)
    "basa_1664x960": dict(T=21, Hg=60, Wg=104, H=12, d=128, q_block=128, kv_block=4,
                          wh=10, ww=10, dy=3, dx=7, ph=4, pw=4, topk=2),
    # the same with 2 x 2 pooling (more global tokens)
    "basa_1664x960_p2": dict(T=21, Hg=60, Wg=104, H=12, d=128, q_block=128, kv_block=4,
                             wh=10, ww=10, dy=3, dx=7, ph=2, pw=2, topk=2),
    # the same with 15 x 26 windows (16 windows of 8,190 tokens: KV block 2)
    "basa_1664x960_w15x26": dict(T=21, Hg=60, Wg=104, H=12, d=128, q_block=128, kv_block=2,
                                 wh=15, ww=26, dy=3, dx=7, ph=4, pw=4, topk=2),
}


def grid_coords(T: int, Hg: int, Wg: int) -> np.ndarray:
    """(N, 3) int64 array of (t, y, x) for tokens in raster order."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int64)


def positional_features(T: int, Hg: int, Wg: int) -> np.ndarray:
    """(N, 16) fp64 sin/cos features of the grid coordinates."""
    coords = grid_coords(T, Hg, Wg).astype(np.float64)
    N = coords.shape[0]
    phi = np.empty((N, 16), dtype=np.float64)
    for f in range(8):
        rate = (np.pi / 2.0) * 2.0 ** (-f / 2.0)
        p = coords[:, f % 3]
        phi[:, 2 * f] = np.sin(rate * p)
        phi[:, 2 * f + 1] = np.cos(rate * p)
    return phi


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE); returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def head_qkv(T: int, Hg: int, Wg: int, d: int, seed: int, h: int, phi=None):
    """One head's (q, k, v) as uint16 bf16 bits, each (N, d)."""
    if d < 16:
        raise ValueError("head dim must be >= 16 for the 16 positional directions")
    N = T * Hg * Wg
    rng = np.random.default_rng([seed, h])
    G = rng.standard_normal((d, d))
    Qf, _ = np.linalg.qr(G)
    u = Qf[:16, :] * np.sqrt(d / 8.0)
    zq = rng.standard_normal((N, d))
    zk = rng.standard_normal((N, d))
    zv = rng.standard_normal((N, d))
    if phi is None:
        phi = positional_features(T, Hg, Wg)
    pos = phi @ u
    q = f64_to_bf16_bits(0.5 * zq + pos)
    k = f64_to_bf16_bits(0.5 * zk + pos)
    v = f64_to_bf16_bits(zv)
    return q, k, v


def _head_job(args):
    T, Hg, Wg, d, seed, h = args
    return head_qkv(T, Hg, Wg, d, seed, h)


def make_qkv(T: int, Hg: int, Wg: int, H: int, d: int, seed: int = 0, B: int = 1,
             workers: int = 1):
    """(q, k, v) uint16 bf16 bit arrays of shape [B, H, N, d].

    Batch b > 0 uses seed ``seed + 1000 * b`` so that batches differ.  With
    ``workers > 1`` heads are drawn in parallel processes (same values: every
    head has its own generator).
    """
    N = T * Hg * Wg
    out = [np.empty((B, H, N, d), dtype=np.uint16) for _ in range(3)]
    jobs = [(T, Hg, Wg, d, seed + 1000 * b, h) for b in range(B) for h in range(H)]
    if workers > 1 and len(jobs) > 1:
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(max_workers=min(workers, len(jobs))) as ex:
            results = list(ex.map(_head_job, jobs))
    else:
        phi = positional_features(T, Hg, Wg)
        results = [head_qkv(T, Hg, Wg, d, s_, h, phi) for (_, _, _, _, s_, h) in jobs]
    for (_, _, _, _, s_, h), (q, k, v) in zip(jobs, results):
        b = (s_ - seed) // 1000
        out[0][b, h], out[1][b, h], out[2][b, h] = q, k, v
    return tuple(out)


def make_config_qkv(name: str, seed: int = 0, heads=None):
    """Inputs of a named workload; ``heads`` optionally limits the head count."""
    c = CONFIGS[name]
    H = c["H"] if heads is None else heads
    return make_qkv(c["T"], c["Hg"], c["Wg"], H, c["d"], seed)


def random_offsets(seed: int, n: int) -> np.ndarray:
    """Arbitrary 44-bit sampling offsets below 2^44 - 2^16 (test inputs)."""
    rng = np.random.default_rng([seed, 7919])
    return rng.integers(0, (1 << 44) - (1 << 16), size=n, dtype=np.int64).astype(np.uint64)
