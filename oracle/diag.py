"""Accuracy diagnostics of a sampling plan: true block attention mass,
retained mass (coverage) of a plan, and output error against dense attention.

Test infrastructure only (see ``oracle/__init__``).

Follows the AB-Attention page (onedev.kr/papers/1521):

* section "무엇과 다른가": the attention mass that an oracle top-k keeps
  grows as the KV blocks shrink (128-token blocks against 4-token blocks);
* section "어떻게 쓰나": SIP's attention error against that of an oracle top-k
  at the same block size;
* section "전제와 한계", ablation paragraph: the variants compared (segment
  means instead of clustering, no pi weighting, uniform sampling, selection
  at the execution tile).

Readings where the pages are silent:

* the attention mass of KV block j for query block i is the mean, over the
  block's queries n, of the dense softmax probability (all Nk keys, scale
  1/sqrt(d) unless given, natural exp) summed over the keys of block j:
  A_ij = (1/|Q_i|) sum_{n in Q_i} sum_{t in B_j} exp(scale q_n . k_t - lse_n);
  the last KV block holds its valid keys only;
* an oracle top-k keeps, per query block (the plan is shared by the block's
  queries), the budget's worth of blocks with the largest A_ij, ties to the
  lowest index;
* the retained mass of a plan is sum_{listed j} A_ij with no 1/pi weight,
  each listed block counted once per entry; entries outside [0, M) are
  skipped;
* attention error = relative Frobenius error ||O - O_dense|| / ||O_dense||
  over one head's outputs.
"""
from __future__ import annotations

import numpy as np


def dense_lse(q: np.ndarray, k: np.ndarray, scale: float | None = None) -> np.ndarray:
    """ln sum_t exp(scale q_n . k_t) for every query row (fp64)."""
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    logits = (q @ k.T) * scale
    m = logits.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))[:, 0]


def block_mass(q, k, q_block: int, kv_block: int, lse=None, scale: float | None = None,
               blocks=None) -> np.ndarray:
    """A (nqb, M) fp64 for one head; q (Nq, d), k (Nk, d) fp64.

    ``lse`` (Nq,) replaces the dense log-normaliser when given (the device
    takes it as an input); ``blocks`` limits the work to the listed query
    blocks (other rows stay NaN).
    """
    Nq, d = q.shape
    Nk = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nqb, M = -(-Nq // q_block), -(-Nk // kv_block)
    A = np.full((nqb, M), np.nan)
    todo = range(nqb) if blocks is None else blocks
    for i in todo:
        r0, r1 = i * q_block, min(Nq, (i + 1) * q_block)
        logits = (q[r0:r1] @ k.T) * scale
        ls = dense_lse(q[r0:r1], k, scale) if lse is None else np.asarray(lse[r0:r1], np.float64)
        p = np.exp(logits - ls[:, None])                 # (n_i, Nk)
        col = p.mean(axis=0)                             # mean over the block's queries
        pad = np.zeros(M * kv_block)
        pad[:Nk] = col
        A[i] = pad.reshape(M, kv_block).sum(axis=1)
    return A


def plan_coverage(A, idx, count) -> np.ndarray:
    """Retained mass per row: sum of A[row, idx[row, e]] for e < count[row]
    (entries outside [0, M) skipped), added in list order in fp64."""
    A = np.asarray(A)
    lead = A.shape[:-1]
    M = A.shape[-1]
    A2 = A.reshape(-1, M)
    idx2 = np.asarray(idx).reshape(A2.shape[0], -1)
    cnt = np.asarray(count).reshape(-1)
    out = np.zeros(A2.shape[0])
    for r in range(A2.shape[0]):
        c = max(0, min(int(cnt[r]), idx2.shape[1]))
        acc = 0.0
        for j in idx2[r, :c]:
            if 0 <= j < M:
                acc += float(A2[r, j])
        out[r] = acc
    return out.reshape(lead)


def output_error(O, ref) -> tuple[float, float]:
    """(sum (O - ref)^2, sum ref^2) over one head, fp64."""
    O = np.asarray(O, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(((O - ref) ** 2).sum()), float((ref ** 2).sum())


def relative_error(O, ref) -> float:
    """||O - ref||_F / ||ref||_F."""
    num, den = output_error(O, ref)
    return float(np.sqrt(num / den))


def oracle_topk(A, budget: int):
    """Per row, the ``budget`` blocks with the largest mass (ties to the
    lowest index), ascending; returns (idx int32, count int32)."""
    A = np.asarray(A, np.float64)
    lead, M = A.shape[:-1], A.shape[-1]
    rows = A.reshape(-1, M)
    s = min(budget, M)
    idx = np.empty((rows.shape[0], s), np.int32)
    for r in range(rows.shape[0]):
        order = np.lexsort((np.arange(M), -rows[r]))
        idx[r] = np.sort(order[:s])
    return idx.reshape(lead + (s,)), np.full(lead, s, np.int32)
