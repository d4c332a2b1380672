"""Sparse attention given a plan: the plain definition, in fp64.

Test infrastructure only (see ``oracle/__init__``).

Follows the AB-Attention page (onedev.kr/papers/1521): the fused pass of
section "전제와 한계" (first paragraph) gathers the sampled KV blocks and runs
softmax attention over them with the logit of every token of block j shifted
by -log pi_ij (section "어떻게 쓰나", where this shift is shown equal to
weighting the numerator and the denominator by 1/pi_ij).  Only a plain
definition is written here: gather the keys, one dense softmax, no tiling and
no online rescaling.

Readings: scale 1/sqrt(d) unless given; no causal mask (full 3D attention of
a video DiT); natural log; the shift applies to every token of the block;
keys with index >= Nk (partial last block, padding) are left out.  The list
format (fixed stride, a per-row count) has two more rules: the count is
clamped to [0, list length], and an entry outside [0, ceil(Nk / kv_block))
names no block and is skipped (the planner marks unused entries with -1 and
a row it could not plan with count -1).  A query block left with no key gets
a zero output and LSE = -inf (the empty sum).

``attn_bwd`` is the gradient of the same definition (the page names a
trainable version, with a backward pass, as future work in its closing
paragraph): with the plan and its shifts held fixed, dQ, dK and dV of
sum(dO * O), each listed occurrence of a block being its own set of keys.
"""
from __future__ import annotations

import numpy as np


def listed_blocks(idx_row, bias_row, count: int, M: int):
    """The entries of one list row that name a block: the first
    min(max(count, 0), L) entries, minus those outside [0, M).  Returns
    (blocks int64, bias fp32); ``bias_row`` None means every shift is 0."""
    row = np.asarray(idx_row).astype(np.int64)
    c = max(0, min(int(count), row.shape[0]))
    bl = row[:c]
    b = np.zeros(c, np.float32) if bias_row is None else np.asarray(bias_row)[:c]
    ok = (bl >= 0) & (bl < M)
    return bl[ok], b[ok]


def gather_keys(blocks: np.ndarray, bias: np.ndarray, kv_block: int, Nk: int):
    """Token indices and per-token logit shift of the listed blocks (each in
    [0, ceil(Nk / kv_block)))."""
    keys = (blocks[:, None].astype(np.int64) * kv_block + np.arange(kv_block)).ravel()
    kb = np.repeat(bias.astype(np.float64), kv_block)
    valid = keys < Nk
    return keys[valid], kb[valid]


def attn_fwd(q, k, v, q_block: int, kv_block: int, idx, bias, count,
             scale: float | None = None, blocks=None):
    """One head.  q (Nq, d), k/v (Nk, d) fp64; idx (nqb, L) int, bias (nqb, L)
    fp32 or None (all pi = 1), count (nqb,) int.

    Returns (O (Nq, d) fp64, LSE (Nq,) fp64 natural log).  ``blocks`` limits the
    work to the listed query blocks (other rows stay NaN).  List entries
    follow ``listed_blocks``; a query block with no key gets O = 0 and
    LSE = -inf.
    """
    Nq, d = q.shape
    Nk = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nqb = -(-Nq // q_block)
    M = -(-Nk // kv_block)
    O = np.full((Nq, d), np.nan)
    lse = np.full(Nq, np.nan)
    todo = range(nqb) if blocks is None else blocks
    for i in todo:
        bl, b = listed_blocks(idx[i], None if bias is None else bias[i], count[i], M)
        keys, kb = gather_keys(bl, b, kv_block, Nk)
        r0, r1 = i * q_block, min(Nq, (i + 1) * q_block)
        if keys.size == 0:
            O[r0:r1] = 0.0
            lse[r0:r1] = -np.inf
            continue
        logits = (q[r0:r1] @ k[keys].T) * scale + kb[None, :]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        den = e.sum(axis=1, keepdims=True)
        O[r0:r1] = (e @ v[keys]) / den
        lse[r0:r1] = (m + np.log(den))[:, 0]
    return O, lse


def dense_attn(q, k, v, scale: float | None = None):
    """Full softmax attention (every key, no shift), fp64."""
    d = q.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    logits = (q @ k.T) * scale
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=1, keepdims=True)
    return (e @ v) / den, (m + np.log(den))[:, 0]


def attn_bwd(q, k, v, dout, q_block: int, kv_block: int, idx, bias, count,
             scale: float | None = None, blocks=None):
    """Gradients of sum(dout * O) for O = attn_fwd(q, k, v, ...), fp64.

    Per query block: gather the listed keys (an entry listed twice is two
    sets of keys), P = softmax(scale q k^T + shift), O = P v, dP = dout v^T,
    D = rowsum(dout * O), dS = P (dP - D); dQ = scale dS k, and dS^T q
    (times scale) and P^T dout are added into dK and dV at the gathered
    token rows.  Returns (dq (Nq, d), dk (Nk, d), dv (Nk, d)).  ``blocks``
    limits the work to the listed query blocks: their dq rows, and dk / dv
    rows complete for keys that no other query block lists.
    """
    Nq, d = q.shape
    Nk = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nqb = -(-Nq // q_block)
    dq = np.zeros((Nq, d))
    dk = np.zeros((Nk, d))
    dv = np.zeros((Nk, d))
    M = -(-Nk // kv_block)
    for i in (range(nqb) if blocks is None else blocks):
        bl, b = listed_blocks(idx[i], None if bias is None else bias[i], count[i], M)
        keys, kb = gather_keys(bl, b, kv_block, Nk)
        if keys.size == 0:
            continue
        r0, r1 = i * q_block, min(Nq, (i + 1) * q_block)
        qi, gi = q[r0:r1], dout[r0:r1]
        logits = (qi @ k[keys].T) * scale + kb[None, :]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        P = e / e.sum(axis=1, keepdims=True)
        O = P @ v[keys]
        dP = gi @ v[keys].T
        D = (gi * O).sum(axis=1, keepdims=True)
        dS = P * (dP - D)
        dq[r0:r1] = scale * (dS @ k[keys])
        np.add.at(dk, keys, scale * (dS.T @ qi))
        np.add.at(dv, keys, P.T @ gi)
    return dq, dk, dv
