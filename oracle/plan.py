"""SIP and top-k sampling-plan oracle.

Test infrastructure only (see ``oracle/__init__``).

Follows the AB-Attention page (onedev.kr/papers/1521), section "어떻게 쓰나"
(SIP): for every query block i, block j gets inclusion probability
pi_ij = min(1, lambda_i * S_ij) with lambda_i chosen so that the pi_ij sum
to the budget s; blocks with pi = 1 are always taken; a systematic sample
draws exactly s distinct blocks, shared by all queries of the block; and the
1/pi weighting becomes a -log pi logit shift.  Top-k (the same budget, no pi
weighting) is the level the ablation paragraph of section "전제와 한계"
equates with SIP minus the weighting.

Numerical definition (this project's reading; the pages give none):

* scores enter as fp32 values (the boundary's dtype), taken exactly;
* if the budget reaches the number M+ of positive scores, every positive
  block is taken with pi = 1 (lambda reported as +inf), count = M+;
* otherwise r = the number of saturated blocks is the smallest r >= 0 with
  (s - r) * S_(r+1) <= T_r, where S_(1) >= S_(2) >= ... are the sorted
  scores and T_r is the exact sum of all but the r largest; the condition is
  evaluated exactly (its truth set is upward closed in r, so the smallest r
  is well defined);
* lambda = (s - r) / T_r with T_r the exact sum correctly rounded to fp64
  and one IEEE fp64 division; pi_j = min(1, lambda * S_j), one IEEE multiply;
* systematic sampling in 44-bit fixed point: Pi_j = floor(pi_j * 2^44),
  C_j = Pi_0 + ... + Pi_j (exact integers), points x_k = U + k * 2^44 for
  k = 0..s-1; block j is drawn when a point lies in [C_{j-1}, C_j);
* output: drawn block indices in ascending order, bias = -ln pi (fp32).

Top-k: the s largest scores, ties to the lowest index, pi = 1, ascending.
"""
from __future__ import annotations

import math

import numpy as np

from .splitmix import UNIT, sampling_offset

SIP = 0
TOPK = 1


def _as_f32_values(S) -> np.ndarray:
    S = np.asarray(S, dtype=np.float64)
    return S.astype(np.float32).astype(np.float64)


def _cond_exact(v: np.ndarray, s: int, r: int) -> bool:
    """(s - r) * v[r] <= sum(v[r:]) exactly; v sorted descending."""
    lhs = (s - r) * float(v[r])          # exact: 24-bit value times an integer < 2^29
    return math.fsum(np.append(v[r:], -lhs)) >= 0.0


def saturated_count(S: np.ndarray, s: int) -> int:
    """Smallest r with the exact saturation condition (needs M+ > s)."""
    v = np.sort(S)[::-1]
    # fp64 estimate first, then exact checks; the condition is monotone in r.
    tail = np.cumsum(v[::-1])[::-1]
    ok = (s - np.arange(s)) * v[:s] <= tail[:s]
    r = int(np.argmax(ok)) if ok.any() else s - 1
    if not _cond_exact(v, s, r):
        lo, hi = r + 1, s - 1                # answer in (r, s - 1]
        while lo < hi:
            mid = (lo + hi) // 2
            if _cond_exact(v, s, mid):
                hi = mid
            else:
                lo = mid + 1
        return lo
    if r > 0 and _cond_exact(v, s, r - 1):
        lo, hi = 0, r - 1
        while lo < hi:
            mid = (lo + hi) // 2
            if _cond_exact(v, s, mid):
                hi = mid
            else:
                lo = mid + 1
        return lo
    return r


def sip_lambda(S: np.ndarray, s: int):
    """(r, T_r, lambda) for one row with more than s positive scores."""
    r = saturated_count(S, s)
    v = np.sort(S)[::-1]
    T = math.fsum(v[r:])
    return r, T, (s - r) / T


def sip_row(S, s: int, U: int):
    """One row: returns (idx int64 ascending, bias fp32, count, lambda)."""
    S = _as_f32_values(S)
    if not np.all(np.isfinite(S)) or np.any(S < 0):
        raise ValueError("scores must be finite and non-negative")
    if not (1 <= s <= S.size):
        raise ValueError("budget out of range")
    pos = np.flatnonzero(S > 0)
    if s >= pos.size:
        return pos.astype(np.int64), np.zeros(pos.size, np.float32), int(pos.size), math.inf
    _, _, lam = sip_lambda(S, s)
    pi = np.minimum(1.0, lam * S)
    Pi = np.floor(pi * float(UNIT)).astype(np.int64)
    Cum = np.cumsum(Pi)
    x = np.int64(U) + np.arange(s, dtype=np.int64) * np.int64(UNIT)
    if Cum[-1] <= x[-1]:
        raise AssertionError("fixed-point mass below the last sampling point")
    j = np.searchsorted(Cum, x, side="right")
    if np.any(np.diff(j) <= 0):
        raise AssertionError("systematic sample not distinct")
    bias = (-np.log(pi[j])).astype(np.float32)
    return j.astype(np.int64), bias, s, lam


def inclusion_probabilities(S, s: int) -> np.ndarray:
    """pi_j of one row (fp64), as used by sip_row."""
    S = _as_f32_values(S)
    pos = np.flatnonzero(S > 0)
    if s >= pos.size:
        return (S > 0).astype(np.float64)
    _, _, lam = sip_lambda(S, s)
    return np.minimum(1.0, lam * S)


def topk_row(S, s: int):
    """Top-s blocks by (-S_j, j); returns (idx ascending, bias zeros, count)."""
    S = _as_f32_values(S)
    if not (1 <= s <= S.size):
        raise ValueError("budget out of range")
    order = np.lexsort((np.arange(S.size), -S))
    sel = np.sort(order[:s]).astype(np.int64)
    return sel, np.zeros(s, np.float32), s


def plan(S, budget: int, mode: int = SIP, seed: int = 0, offsets=None, row_base: int = 0):
    """Plan for a stack of rows S (..., M).

    Row r (flattened, plus ``row_base``) uses ``offsets[r]`` when given, else
    the seeded offset of that row.  Returns idx (..., budget) int32 padded
    with -1, bias (..., budget) fp32 padded with 0, count (...) int32,
    lam (...) fp64.
    """
    S = np.asarray(S, dtype=np.float64)
    lead = S.shape[:-1]
    rows = S.reshape(-1, S.shape[-1])
    n = rows.shape[0]
    idx = np.full((n, budget), -1, np.int32)
    bias = np.zeros((n, budget), np.float32)
    cnt = np.zeros(n, np.int32)
    lam = np.zeros(n, np.float64)
    for r in range(n):
        if mode == SIP:
            U = int(offsets[r]) if offsets is not None else sampling_offset(seed, row_base + r)
            j, b, c, lm = sip_row(rows[r], budget, U)
        else:
            j, b, c = topk_row(rows[r], budget)
            lm = 0.0
        idx[r, :c], bias[r, :c], cnt[r], lam[r] = j, b, c, lm
    return (idx.reshape(lead + (budget,)), bias.reshape(lead + (budget,)),
            cnt.reshape(lead), lam.reshape(lead))
