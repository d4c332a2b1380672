"""Pins of the SIP / top-k plan oracle: exact rational brute force, closed
forms, sampling invariants, the published SplitMix64 outputs and the
operating points printed on the AB-Attention page."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import plan as opl
from oracle.splitmix import OFFSET_LIMIT, UNIT, sampling_offset, splitmix64


def test_splitmix64_published_outputs(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "splitmix64_seed1234567.json")))
    got = [splitmix64(g["seed"], i) for i in range(len(g["outputs"]))]
    assert got == [int(x) for x in g["outputs"]]


def test_offsets_in_range():
    for seed in (0, 1, 2**63 + 5):
        for row in range(0, 5000, 7):
            u = sampling_offset(seed, row)
            assert 0 <= u < OFFSET_LIMIT


def _row(rng, M, zeros=0, ties=0):
    S = rng.gamma(0.3, size=M)
    S /= S.sum()
    if ties:
        S[rng.integers(0, M, ties)] = S[rng.integers(0, M)]
    if zeros:
        S[rng.integers(0, M, zeros)] = 0.0
    return S.astype(np.float32).astype(np.float64)


def _saturated_count_linear_exact(S, s):
    """Linear scan with exact rational arithmetic (brute force)."""
    v = sorted((Fraction(float(x)) for x in S), reverse=True)
    for r in range(s):
        if (s - r) * v[r] <= sum(v[r:], Fraction(0)):
            return r
    raise AssertionError


def _lambda_by_bisection(S, s):
    """Root of sum_j min(1, lam S_j) = s by exact rational bisection."""
    Sf = [Fraction(float(x)) for x in S if x > 0]
    lo, hi = Fraction(0), Fraction(1) / min(Sf) * 2

    def f(lam):
        return sum(min(Fraction(1), lam * x) for x in Sf)

    for _ in range(200):
        mid = (lo + hi) / 2
        if f(mid) < s:
            lo = mid
        else:
            hi = mid
    return float((lo + hi) / 2)


@pytest.mark.parametrize("seed", range(12))
def test_saturated_count_and_lambda_brute_force(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(20, 90))
    S = _row(rng, M, zeros=int(rng.integers(0, 4)), ties=int(rng.integers(0, 6)))
    npos = int((S > 0).sum())
    s = int(rng.integers(1, npos))
    r, T, lam = opl.sip_lambda(S, s)
    assert r == _saturated_count_linear_exact(S, s)
    assert T == float(sum((Fraction(float(x)) for x in sorted(S, reverse=True)[r:]), Fraction(0)))
    assert lam == (s - r) / T
    assert math.isclose(lam, _lambda_by_bisection(S, s), rel_tol=1e-14)


@pytest.mark.parametrize("seed", range(8))
def test_inclusion_probabilities_sum_to_budget(seed):
    rng = np.random.default_rng(100 + seed)
    S = _row(rng, 500, zeros=3)
    for s in (1, 17, 100, 480):
        pi = opl.inclusion_probabilities(S, s)
        assert abs(math.fsum(pi) - s) <= 1e-12 * s
        assert np.all(pi[S > 0] > 0) and np.all(pi <= 1.0) and np.all(pi[S == 0] == 0)


def test_equal_scores_give_uniform_pi_and_even_spacing():
    M, s = 1024, 64
    S = np.full(M, 1.0 / M)
    pi = opl.inclusion_probabilities(S, s)
    assert np.all(pi == s / M)
    for U in (0, 12345, OFFSET_LIMIT - 1):
        idx, bias, cnt, lam = opl.sip_row(S, s, U)
        assert cnt == s
        d = np.diff(idx)
        assert np.all(d == M // s)
        np.testing.assert_allclose(bias, -np.log(s / M), rtol=1e-7)


def test_budget_covering_all_positive_blocks():
    S = np.array([0.0, 0.5, 0.0, 0.25, 0.25])
    idx, bias, cnt, lam = opl.sip_row(S, 3, 0)
    assert list(idx) == [1, 3, 4] and cnt == 3 and lam == math.inf
    assert np.all(bias == 0)
    idx, bias, cnt, lam = opl.sip_row(S, 5, 0)
    assert list(idx) == [1, 3, 4] and cnt == 3


@pytest.mark.parametrize("seed", range(6))
def test_sample_is_exact_distinct_and_keeps_saturated_blocks(seed):
    rng = np.random.default_rng(200 + seed)
    S = _row(rng, 3000, zeros=20, ties=30)
    for s in (5, 300, 2000):
        pi = opl.inclusion_probabilities(S, s)
        for U in (0, int(rng.integers(0, OFFSET_LIMIT)), OFFSET_LIMIT - 1):
            idx, bias, cnt, lam = opl.sip_row(S, s, U)
            assert cnt == s and len(idx) == s
            assert np.all(np.diff(idx) > 0)
            assert np.all(S[idx] > 0)
            assert set(np.flatnonzero(pi == 1.0)) <= set(idx.tolist())
            np.testing.assert_allclose(bias, -np.log(pi[idx]), rtol=1e-6, atol=1e-7)


def test_inclusion_frequency_over_offset_sweep():
    """Over G equally spaced offsets the inclusion count of block j is
    floor-or-ceil of Pi_j * G / 2^44 (first-order inclusion = pi)."""
    rng = np.random.default_rng(7)
    S = _row(rng, 200, zeros=2)
    s, G = 40, 512
    pi = opl.inclusion_probabilities(S, s)
    Pi = np.floor(pi * float(UNIT)).astype(np.int64)
    hits = np.zeros(200, np.int64)
    for g in range(G):
        idx, _, _, _ = opl.sip_row(S, s, (g * UNIT) // G)
        hits[idx] += 1
    expect = Pi * G / float(UNIT)
    assert np.all(np.abs(hits - expect) <= 1.0 + 1e-9)


def test_horvitz_thompson_total_is_unbiased_over_offsets():
    rng = np.random.default_rng(8)
    S = _row(rng, 300, zeros=0)
    x = rng.standard_normal(300) * S * 50
    s, G = 60, 2048
    pi = opl.inclusion_probabilities(S, s)
    ests = []
    for g in range(G):
        idx, bias, _, _ = opl.sip_row(S, s, (g * UNIT) // G)
        ests.append(np.sum(x[idx] / pi[idx]))
    bound = np.sum(np.abs(x) / pi) / G + 1e-9
    assert abs(np.mean(ests) - x.sum()) <= bound


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_stable_sort(seed):
    rng = np.random.default_rng(300 + seed)
    S = _row(rng, 150, zeros=10, ties=40)
    for s in (1, 8, 77, 150):
        idx, bias, cnt = opl.topk_row(S, s)
        ref = sorted(sorted(range(150), key=lambda j: (-float(S[j]), j))[:s])
        assert list(idx) == ref and cnt == s and np.all(bias == 0)


def test_plan_uses_seeded_offsets_per_row():
    rng = np.random.default_rng(9)
    S = np.stack([_row(rng, 64) for _ in range(6)]).reshape(2, 3, 64)
    idx, bias, cnt, lam = opl.plan(S, 10, opl.SIP, seed=42)
    for r in range(6):
        want, _, _, _ = opl.sip_row(S.reshape(6, 64)[r], 10, sampling_offset(42, r))
        assert list(idx.reshape(6, 10)[r]) == list(want)


def test_budgets_reproduce_page_sparsity(golden_dir):
    """s = floor((1 - p) M) reproduces the page's sparsity and computed share
    at the Wan2.1 720p (M = 18900) and HunyuanVideo 720p (M = 29700) shapes."""
    g = json.load(open(os.path.join(golden_dir, "ab_attention_operating_points.json")))
    for M, key in ((18900, "wan2.1"), (29700, "hunyuanvideo")):
        p = g["sparsity_pct"][key] / 100
        s = math.floor((1 - p) * M)
        assert round(100 * (1 - s / M), 2) == g["sparsity_pct"][key]
        assert (s * g["kv_block"]) % g["q_block"] == 0   # whole 128-key tiles
    s = math.floor((1 - 0.9235) * 29700)
    assert round(100 * s / 29700, 2) == g["computed_pct"]["hunyuanvideo"]
    assert math.floor((1 - 0.8916) * 18900) == 2048 and s == 2272


def _worst_uniform_budget(M):
    """The budget s whose uniform row (all scores equal) loses the most
    fixed-point mass to the floors: pi = s / M for every block, and
    s 2^44 - M floor(pi 2^44) is largest."""
    s = np.arange(1, M, dtype=np.int64)
    lam = s.astype(np.float64) / M                      # one IEEE division, as the oracle
    Pi = np.floor(lam * float(UNIT)).astype(np.int64)   # exact scaling by 2^44
    deficit = s * UNIT - M * Pi
    k = int(np.argmax(deficit))
    return int(s[k]), int(deficit[k])


def test_exactly_s_blocks_up_to_the_sip_row_limit():
    """The floors of Pi_j lose less than one unit each and fp64 rounding
    little more, so the fixed-point mass C_M stays above the last point
    U + (s - 1) 2^44 for every offset U < 2^44 - 2^16 while M <= 65,024
    (the limit the boundary enforces for SIP rows): the worst uniform row at
    that M, with the largest offset, still draws exactly s blocks.  At
    M = 2^17 + 1 the worst uniform row loses more than 2^16 units, and the
    largest offset's last point falls past C_M."""
    Umax = UNIT - (1 << 16) - 1
    M = 65024
    s, deficit = _worst_uniform_budget(M)
    assert (1 << 15) < deficit < (1 << 16)
    j, _, c, _ = opl.sip_row(np.ones(M), s, Umax)
    assert c == s and len(np.unique(j)) == s
    M = (1 << 17) + 1
    s, deficit = _worst_uniform_budget(M)
    assert deficit > (1 << 16)
    with pytest.raises(AssertionError):
        opl.sip_row(np.ones(M), s, Umax)
