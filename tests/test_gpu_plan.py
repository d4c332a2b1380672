"""GPU parity of bsa_sip_plan against the oracle: indices and counts bit-exact,
lambda bitwise, bias within 2 fp32 ulp, on the same fp32 scores and the same
offsets (seeded or explicit)."""
import numpy as np
import pytest

from oracle import plan as opl
from oracle import select as osel
from oracle.splitmix import OFFSET_LIMIT
from synth import CONFIGS, make_qkv, random_offsets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def _rows(rng, n, M, zeros=0, ties=0):
    S = rng.gamma(0.3, size=(n, M))
    for r in range(n):
        if ties:
            S[r, rng.integers(0, M, ties)] = S[r, rng.integers(0, M)]
        if zeros:
            S[r, rng.integers(0, M, zeros)] = 0.0
    S /= S.sum(axis=1, keepdims=True)
    return S.astype(np.float32)


def _gpu_plan(env, S32, budget, mode, seed=0, offsets=None):
    bsa, g, torch = env
    t = torch.from_numpy(np.ascontiguousarray(S32)).cuda()
    off = None if offsets is None else torch.from_numpy(offsets.astype(np.int64)).cuda()
    idx, bias, cnt, lam = bsa.bsa_sip_plan(t, budget, mode, seed=seed, offsets=off,
                                           want_lambda=True)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), bias.cpu().numpy(), cnt.cpu().numpy(), lam.cpu().numpy()


def _compare(S32, got, want, what):
    gi, gb, gc, gl = got
    wi, wb, wc, wl = want
    bad = np.flatnonzero((gi != wi).any(axis=-1).ravel() | (gc != wc).ravel())
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first {bad[:5]}"
    assert np.array_equal(gl.view(np.int64), wl.view(np.int64)) or \
        np.array_equal(gl, wl), f"{what}: lambda differs"
    ulp = np.abs(gb.view(np.int32).astype(np.int64) - wb.view(np.int32).astype(np.int64))
    close = (ulp <= 2) | (np.abs(gb) + np.abs(wb) == 0)
    assert close.all(), f"{what}: bias off by {ulp.max()} ulp"


@pytest.mark.parametrize("M,s,mode", [
    (32, 8, opl.TOPK), (100, 7, opl.SIP), (1000, 100, opl.SIP), (1000, 100, opl.TOPK),
    (8190, 887, opl.SIP), (18900, 2048, opl.SIP), (29700, 2272, opl.SIP),
    (29700, 2272, opl.TOPK), (5000, 4990, opl.SIP), (333, 1, opl.SIP),
])
def test_plan_matches_oracle_random_rows(env, M, s, mode):
    bsa, g, torch = env
    g.say(f"case plan random M={M} s={s} mode={mode}")
    rng = np.random.default_rng(M + s + mode)
    S = _rows(rng, 24, M, zeros=M // 50, ties=M // 40).reshape(1, 2, 12, M)
    got = _gpu_plan(env, S, s, mode, seed=123)
    want = opl.plan(S, s, mode, seed=123)
    _compare(S, got, want, f"M={M} s={s}")


@pytest.mark.parametrize("mode", [opl.SIP, opl.TOPK])
def test_plan_structured_fuzz(env, mode):
    """Many small rows built to sit on the search's edge cases: values from a
    few powers of two (so sums and products are exact and equalities
    happen), repeated values, zeros, one value nudged a few ulps off its
    neighbour, and budgets from 1 up to the row length."""
    bsa, g, torch = env
    g.say(f"case plan structured fuzz mode={mode}")
    for M in (5, 9, 17, 40, 96, 300):
        H = max(1, M // 8)  # size of the head of large values (second family)
        for s in sorted({1, 2, 3, H // 2 + 1, H, H + 1, H + 3, 2 * H, M // 4 + 1, M // 2, M - 1, M}):
            rng = np.random.default_rng(M * 1009 + s * 7 + mode)
            rows = []
            for r in range(16):
                if r % 2 == 0:  # spread powers of two
                    v = 2.0 ** -rng.integers(1, 12, M).astype(np.float64)
                else:           # a head of large values over a tail of small ones
                    v = 2.0 ** -rng.integers(6, 15, M).astype(np.float64)
                    v[rng.permutation(M)[:H]] = 2.0 ** -rng.integers(1, 4, H)
                v[rng.random(M) < 0.1] = 0.0
                k = rng.integers(0, M)  # one value a few ulps above another
                if v[k] > 0:
                    v[k] = np.float64(np.float32(v[rng.integers(0, M)]) *
                                      np.float32(1 + rng.integers(1, 4) * 2.0 ** -23))
                rows.append(v)
            S = np.stack(rows).astype(np.float32).reshape(1, 2, 8, M)
            got = _gpu_plan(env, S, s, mode, seed=M * 31 + s)
            want = opl.plan(S, s, mode, seed=M * 31 + s)
            _compare(S, got, want, f"fuzz M={M} s={s}")


def test_plan_explicit_offsets(env):
    bsa, g, torch = env
    g.say("case plan explicit offsets")
    rng = np.random.default_rng(5)
    S = _rows(rng, 16, 2000, zeros=10).reshape(1, 1, 16, 2000)
    off = random_offsets(3, 16)
    off[0], off[1] = 0, OFFSET_LIMIT - 1
    got = _gpu_plan(env, S, 300, opl.SIP, offsets=off)
    want = opl.plan(S, 300, opl.SIP, offsets=off)
    _compare(S, got, want, "explicit offsets")


def test_plan_exact_ties_and_special_rows(env):
    """Rows whose saturation test holds with equality (the exact-sum path),
    equal scores, budget >= positives, all-zero and invalid rows."""
    bsa, g, torch = env
    g.say("case plan special rows")
    M = 66
    rows = []
    a, y = 2.0 ** -5, 2.0 ** -10
    r0 = np.array([a, a] + [y] * 64)                 # 4a = 2a + 64y: equality at r = 0
    rows.append(r0)
    r1 = np.zeros(M); r1[:64] = 1 / 64               # equal scores
    rows.append(r1)
    r2 = np.zeros(M); r2[[3, 9, 10]] = [0.5, 0.25, 0.25]   # 3 positives < budget
    rows.append(r2)
    r3 = np.array([3 * a, a, a] + [y] * 63)          # mixed with an exact boundary
    rows.append(r3)
    S = np.stack(rows).astype(np.float32).reshape(1, 1, 4, M)
    got = _gpu_plan(env, S, 4, opl.SIP, seed=9)
    want = opl.plan(S, 4, opl.SIP, seed=9)
    _compare(S, got, want, "special rows")
    assert got[2][0, 0, 2] == 3 and np.isinf(got[3][0, 0, 2])
    zero = np.zeros((1, 1, 1, 40), np.float32)
    got = _gpu_plan(env, zero, 5, opl.TOPK)
    assert list(got[0][0, 0, 0]) == [0, 1, 2, 3, 4]
    bad = np.ones((1, 1, 3, 40), np.float32)
    bad[0, 0, 0, 7] = np.nan
    bad[0, 0, 1, 3] = -1.0
    bad[0, 0, 2, 0] = np.inf
    for mode in (opl.SIP, opl.TOPK):
        gi, gb, gc, gl = _gpu_plan(env, bad, 5, mode)
        assert np.all(gc == -1) and np.all(gi == -1)


def test_plan_threshold_inside_the_final_bracket(env):
    """Rows whose threshold x* is a row value strictly below the maximum, so
    the search ends with row values inside its bracket and resolves them
    one by one: cond holding with equality at x* = c (undecided under the
    double-double margin, decided exactly), the same with x* repeated, and
    200 distinct values packed within 2e-4 of each other around x* (more
    values in the bracket than are resolved directly, so bisection narrows
    it first)."""
    bsa, g, torch = env
    g.say("case plan threshold inside the final bracket")
    c, y, b = 2.0 ** -6, 3 * 2.0 ** -12, 10 * 2.0 ** -6   # 3c = 64 y: equality at x* = c
    cases = [(np.array([b, c] + [y] * 64), 5),             # r = 1, T_r = 4c
             (np.array([b, c, c] + [y] * 64 + [0.0]), 6)]  # r = 1, x* = c twice
    clus = 2.0 ** -8 * (1 + np.arange(200) * 2.0 ** -20)
    w = np.frombuffer(np.uint32(964319093).tobytes(), np.float32)[0]  # 109 of the 200 saturate
    cases.append((np.concatenate([clus, np.full(1800, w)]), 310))
    clus2 = 2.0 ** -8 * (1 + np.arange(200) * 2.0 ** -14)
    cases.append((np.concatenate([clus2, np.full(1800, 2.0 ** -12)]), 312))
    # max S just above T / s (within 2^-20): the test at the maximum fails and
    # the bracket starts at the smallest positive value, which is repeated
    cases.append((np.array([1.0, 1.0 - 2.0 ** -22] + [2.0 ** -40] * 3), 2))
    cases.append((np.concatenate([[1.0], 1.0 - np.arange(1, 6) * 2.0 ** -22, np.full(20, 2.0 ** -40)]), 6))
    for row, s in cases:
        S = row.astype(np.float32)
        assert np.array_equal(S.astype(np.float64), row)   # every value is an fp32
        S = S.reshape(1, 1, 1, -1)
        got = _gpu_plan(env, S, s, opl.SIP, seed=4)
        want = opl.plan(S, s, opl.SIP, seed=4)
        _compare(S, got, want, f"bracket row M={S.shape[-1]} s={s}")
    got = _gpu_plan(env, np.array([b, c] + [y] * 64, np.float32).reshape(1, 1, 1, -1), 5, opl.SIP)
    assert got[3][0, 0, 0] == 64.0 and got[2][0, 0, 0] == 5   # lambda = (5 - 1) / (4c)


def test_plan_sum_on_rounding_midpoints(env):
    """Rows whose T_r lies exactly on, or just off, a midpoint between two
    fp64 values: lambda = 1 / RN(T_r) must still match the oracle's
    correctly rounded sum bit for bit (ties to even)."""
    bsa, g, torch = env
    g.say("case plan T_r on fp64 midpoints")
    M = 8
    rows = []
    for tail in ([2.0 ** -53], [3 * 2.0 ** -53], [2.0 ** -53, 2.0 ** -80], [2.0 ** -53, 2.0 ** -100],
                 [2.0 ** -24, 2.0 ** -77], [5 * 2.0 ** -53]):
        r = np.zeros(M)
        r[0] = 1.0
        r[1:1 + len(tail)] = tail
        rows.append(r)
    S = np.stack(rows).astype(np.float32)
    assert np.array_equal(S.astype(np.float64), np.stack(rows))   # every value is an fp32
    S = S.reshape(1, 1, len(rows), M)
    got = _gpu_plan(env, S, 1, opl.SIP, seed=3)
    want = opl.plan(S, 1, opl.SIP, seed=3)
    _compare(S, got, want, "midpoint rows")
    assert got[3][0, 0, 0] == 1.0 and got[3][0, 0, 1] == 1.0 / (1.0 + 2.0 ** -51)


def test_plan_on_selector_scores_full_rows(env):
    """Rows of real selector output (oracle scores of one Wan2.1-14B 720p
    head, rounded to fp32): 48 rows of M = 18,900 at budget 2048."""
    bsa, g, torch = env
    c = CONFIGS["wan14b_720p"]
    g.say("case plan on selector scores wan14b")
    qb, kb, _ = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    S, _, _ = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, 4, 8, 1)
    rows = np.r_[0:24, 567:591]
    S32 = S[rows].astype(np.float32)[None, None]
    got = _gpu_plan(env, S32, 2048, opl.SIP, seed=0)
    want = opl.plan(S32, 2048, opl.SIP, seed=0)
    _compare(S32, got, want, "selector rows")
    assert np.all(got[2] == 2048)


def test_plan_deterministic(env):
    bsa, g, torch = env
    g.say("case plan determinism")
    S = _rows(np.random.default_rng(1), 8, 3000).reshape(1, 1, 8, 3000)
    a1 = _gpu_plan(env, S, 400, opl.SIP, seed=4)
    a2 = _gpu_plan(env, S, 400, opl.SIP, seed=4)
    for x, y in zip(a1, a2):
        assert np.array_equal(x, y)


def test_plan_status_word(env):
    """The optional status word: BSA_OK after a call on valid rows, and
    BSA_ERR_NONFINITE after a call with one bad row among good ones (the
    bad row gets count -1, the good rows their plans); it is reset by every
    call, so a good call after a bad one reads BSA_OK again."""
    bsa, g, torch = env
    g.say("case plan status word")
    rng = np.random.default_rng(5)
    S = _rows(rng, 6, 500).reshape(1, 2, 3, 500)
    st = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    t = torch.from_numpy(S.copy()).cuda()
    for mode in (opl.SIP, opl.TOPK):
        bsa.bsa_sip_plan(t, 20, mode, seed=1, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == bsa.OK
        bad = S.copy()
        bad[0, 1, 2, 17] = np.nan if mode == opl.SIP else -0.5
        tb = torch.from_numpy(bad).cuda()
        idx, _, cnt, _ = bsa.bsa_sip_plan(tb, 20, mode, seed=1, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == bsa.ERR_NONFINITE
        c = cnt.cpu().numpy()
        assert c[0, 1, 2] == -1 and (np.delete(c.ravel(), 5) == 20).all()
        want = opl.plan(S[0, 0], 20, mode, seed=1)      # head 0: rows 0..2, all valid
        assert np.array_equal(idx.cpu().numpy()[0, 0], want[0])
        bsa.bsa_sip_plan(t, 20, mode, seed=1, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == bsa.OK


def test_plan_at_the_sip_row_limit(env):
    """The longest SIP row the boundary accepts (65,024 blocks, the row
    re-read from memory since it exceeds the LDS) with the budget that loses
    the most fixed-point mass to the floors and the largest offset: exactly s
    blocks, equal to the oracle's.  One block longer is refused."""
    bsa, g, torch = env
    M = 65024
    s_all = np.arange(1, M, dtype=np.int64)
    Pi = np.floor((s_all.astype(np.float64) / M) * float(1 << 44)).astype(np.int64)
    s = int(s_all[np.argmax(s_all * (1 << 44) - M * Pi)])
    g.say(f"case plan at the SIP row limit M={M} s={s}")
    S = np.ones((1, 1, 2, M), np.float32)
    S[0, 0, 1, ::7] = 0.5
    off = np.array([OFFSET_LIMIT - 1, OFFSET_LIMIT - 1], np.uint64)
    got = _gpu_plan(env, S, s, opl.SIP, offsets=off)
    want = opl.plan(S, s, opl.SIP, offsets=off)
    _compare(S, got, want, "row limit")
    assert (got[2] == s).all()
    with pytest.raises(bsa.BsaError):
        bsa.bsa_sip_plan(torch.ones((1, 1, 1, M + 1), device="cuda"), 10, bsa.PLAN_SIP)
