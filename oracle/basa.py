"""BASA-structured attention oracle, written from the definition (no lists).

Test infrastructure only (see ``oracle/__init__``).

Follows the BASA page (onedev.kr/papers/688):

* section "어떻게 동작하나": the latent grid is cyclically shifted by -Delta
  and cut into non-overlapping w_h x w_w spatial windows, each window keeping
  every frame; softmax attention runs inside each window; the result is
  shifted back.  The same section gives the per-layer offset schedule
  a_i = (i * delta) mod w, delta = max(1, floor(w / L)), with the first and
  second halves interleaved (worked example: w = 8, L = 4 turns (0, 2, 4, 6)
  into (0, 4, 2, 6));
* section "무엇과 다른가": keys and values are mean-pooled spatially per frame
  (time kept) into a global memory G appended to every window's keys and
  values only; each query window i gets a descriptor q_i (mean query) and
  every candidate window j a key descriptor k_j, relevance
  s_ij = q_i . k_j / sqrt(d), and the top-K candidates R_i contribute their
  raw keys and values; window i attends to W_i U R_i U G; queries and output
  keep their length.

Readings where the page is silent: roll by -Delta means y' = (y - dy) mod Hg,
x' = (x - dx) mod Wg; a ragged last window row/column keeps its smaller
size; the candidate set is every other window; key descriptor = mean key of
the window over all frames; ties go to the lowest window index; pooling is
on the unshifted grid with non-overlapping p_h x p_w cells (a ragged cell
averages its valid tokens); G is appended to every window with no dedupe.

The routing is a discrete decision, so the window means and their dot
products are evaluated in fp32 in one stated order (the HIP kernel uses the
same): a window sum runs over the window's tokens in window-local order
(frame, then shifted row, then shifted column, ascending), one rounding per
add, then one IEEE division by the token count; the dot product runs over
dims 0..d-1 ascending with a rounded multiply and a rounded add.  Ranking
uses the unscaled dot product (1/sqrt(d) > 0 does not change the order).
Attention itself is fp64.
"""
from __future__ import annotations

import numpy as np


def window_grid(Hg: int, Wg: int, wh: int, ww: int):
    """Number of window rows and columns of the shifted grid."""
    return -(-Hg // wh), -(-Wg // ww)


def window_members(T: int, Hg: int, Wg: int, wh: int, ww: int, dy: int, dx: int):
    """Token indices of every window, in window-local order.

    Window id = a * nwx + b for window row a and column b of the shifted grid.
    """
    nwy, nwx = window_grid(Hg, Wg, wh, ww)
    out = []
    for a in range(nwy):
        for b in range(nwx):
            ys = (np.arange(a * wh, min(Hg, (a + 1) * wh)) + dy) % Hg
            xs = (np.arange(b * ww, min(Wg, (b + 1) * ww)) + dx) % Wg
            t, y, x = np.meshgrid(np.arange(T), ys, xs, indexing="ij")
            out.append(((t * Hg + y) * Wg + x).ravel().astype(np.int64))
    return out


def window_of_token(T: int, Hg: int, Wg: int, wh: int, ww: int, dy: int, dx: int):
    """Window id of every token (raster order)."""
    nwy, nwx = window_grid(Hg, Wg, wh, ww)
    N = T * Hg * Wg
    n = np.arange(N)
    y = (n // Wg) % Hg
    x = n % Wg
    return (((y - dy) % Hg) // wh) * nwx + ((x - dx) % Wg) // ww


def _seq_mean_f32(rows: np.ndarray) -> np.ndarray:
    acc = np.zeros(rows.shape[1], np.float32)
    for r in rows:
        acc = acc + r
    return acc / np.float32(rows.shape[0])


def _seq_dot_f32(a: np.ndarray, b: np.ndarray) -> np.float32:
    acc = np.float32(0.0)
    for kk in range(a.shape[0]):
        acc = np.float32(acc + np.float32(a[kk] * b[kk]))
    return acc


def window_descriptors(x32: np.ndarray, members):
    """fp32 mean of x over every window's tokens (window-local order)."""
    return np.stack([_seq_mean_f32(x32[m]) for m in members])


def route(q32: np.ndarray, k32: np.ndarray, members, topk: int):
    """(nW, topk) routed windows: top-k of q_i . k_j over j != i, ties lowest j."""
    qd = window_descriptors(q32, members)
    kd = window_descriptors(k32, members)
    nW = len(members)
    out = np.empty((nW, topk), np.int64)
    for i in range(nW):
        sc = np.array([_seq_dot_f32(qd[i], kd[j]) for j in range(nW)], dtype=np.float64)
        cand = np.array([j for j in range(nW) if j != i])
        order = np.lexsort((cand, -sc[cand]))
        out[i] = cand[order[:topk]]
    return out


def pooled_memory(x64: np.ndarray, T: int, Hg: int, Wg: int, ph: int, pw: int):
    """(T * ceil(Hg/ph) * ceil(Wg/pw), d) fp64 spatial cell means, raster order."""
    d = x64.shape[1]
    g = x64.reshape(T, Hg, Wg, d)
    py, px = -(-Hg // ph), -(-Wg // pw)
    out = np.empty((T, py, px, d))
    for a in range(py):
        for b in range(px):
            out[:, a, b] = g[:, a * ph:(a + 1) * ph, b * pw:(b + 1) * pw].mean(axis=(1, 2))
    return out.reshape(-1, d)


def basa_attn(q_bits, k_bits, v_bits, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk,
              windows=None, routes=None):
    """One head of BASA-structured attention, fp64.  Inputs are bf16 bit arrays.

    Returns (O (N, d) fp64 with NaN outside ``windows``, routes (nW, topk)).
    """
    from synth import bf16_bits_to_f32, bf16_bits_to_f64
    q32, k32 = bf16_bits_to_f32(q_bits), bf16_bits_to_f32(k_bits)
    q, k, v = (bf16_bits_to_f64(x) for x in (q_bits, k_bits, v_bits))
    N, d = q.shape
    members = window_members(T, Hg, Wg, wh, ww, dy, dx)
    if routes is None:
        routes = route(q32, k32, members, topk)
    gk = pooled_memory(k, T, Hg, Wg, ph, pw)
    gv = pooled_memory(v, T, Hg, Wg, ph, pw)
    O = np.full((N, d), np.nan)
    scale = 1.0 / np.sqrt(d)
    todo = range(len(members)) if windows is None else windows
    for w in todo:
        keys = np.concatenate([members[w]] + [members[j] for j in routes[w]])
        kk = np.concatenate([k[keys], gk])
        vv = np.concatenate([v[keys], gv])
        rows = members[w]
        logits = (q[rows] @ kk.T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        O[rows] = (e @ vv) / e.sum(axis=1, keepdims=True)
    return O, routes


def shift_offsets(w: int, L: int):
    """Per-layer window offsets: a_i = (i * delta) mod w, delta = max(1, w // L),
    reordered by interleaving the first and the second half (K = ceil(L / 2)).
    """
    delta = max(1, w // L)
    a = [(i * delta) % w for i in range(L)]
    K = -(-L // 2)
    out = []
    for i in range(K):
        out.append(a[i])
        if K + i < L:
            out.append(a[K + i])
    return out


def layer_step_shift(b_h, b_w, c_h, c_w, l: int, s: int, wh: int, ww: int):
    """Delta_{l,s} = ((b_l^h + c_s^h) mod w_h, (b_l^w + c_s^w) mod w_w)."""
    return ((b_h[l] + c_h[s]) % wh, (b_w[l] + c_w[s]) % ww)
