"""Pins of the attention oracle: dense reduction (torch SDPA, fp64 CPU),
the -log pi shift versus explicit 1/pi weighting, Horvitz-Thompson
unbiasedness of numerator and denominator, and key masking."""
import numpy as np
import pytest
import torch

from oracle import attn as oat
from oracle import plan as opl
from oracle.splitmix import UNIT
from synth import bf16_bits_to_f64, make_qkv


def _head(T, Hg, Wg, d, seed=0):
    q, k, v = make_qkv(T, Hg, Wg, 1, d, seed)
    return tuple(bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))


@pytest.mark.parametrize("kv_block", [1, 4, 64, 128])
def test_all_blocks_pi_one_is_dense_attention(kv_block):
    q, k, v = _head(1, 16, 24, 64, seed=1)
    N = q.shape[0]
    M = -(-N // kv_block)
    nqb = -(-N // 128)
    idx = np.tile(np.arange(M), (nqb, 1))
    cnt = np.full(nqb, M)
    O, lse = oat.attn_fwd(q, k, v, 128, kv_block, idx, None, cnt)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
    np.testing.assert_allclose(O, ref, atol=1e-12, rtol=1e-10)
    lref = torch.logsumexp(torch.from_numpy(q @ k.T / 8.0), dim=-1).numpy()
    np.testing.assert_allclose(lse, lref, rtol=1e-13)


def test_shift_equals_inverse_probability_weighting():
    q, k, v = _head(1, 16, 32, 64, seed=2)
    N, d = q.shape
    kvb, M, s = 4, N // 4, 40
    rng = np.random.default_rng(3)
    S = rng.gamma(0.5, size=(4, M))
    S /= S.sum(axis=1, keepdims=True)
    idx, bias, cnt, _ = opl.plan(S, s, opl.SIP, seed=5)
    O, _ = oat.attn_fwd(q, k, v, 128, kvb, idx, bias, cnt)
    for i in range(4):
        pi = opl.inclusion_probabilities(S[i], s)
        # weights 1/pi from the stored (fp32) shift, then from the exact pi
        for inv_pi, tol in ((lambda t, j: np.exp(np.float64(bias[i, t])), 1e-12),
                            (lambda t, j: 1.0 / pi[j], 1e-6)):
            num = np.zeros((128, d)); den = np.zeros((128, 1))
            for t, j in enumerate(idx[i, :cnt[i]]):
                e = np.exp(q[i * 128:(i + 1) * 128] @ k[j * 4:(j + 1) * 4].T / np.sqrt(d))
                num += e @ v[j * 4:(j + 1) * 4] * inv_pi(t, j)
                den += e.sum(axis=1, keepdims=True) * inv_pi(t, j)
            np.testing.assert_allclose(O[i * 128:(i + 1) * 128], num / den, rtol=0, atol=tol)


def test_ht_numerator_and_denominator_unbiased_over_offsets():
    """Mean over an offset sweep of the 1/pi-weighted numerator and
    denominator tends to the dense ones (the ratio itself is not asserted)."""
    q, k, v = _head(1, 8, 16, 32, seed=4)
    d = q.shape[1]
    kvb, M, s, G = 4, 32, 8, 1024
    qrow = q[:4]
    e_blocks = [np.exp(qrow @ k[j * 4:(j + 1) * 4].T / np.sqrt(d)) for j in range(M)]
    dense_num = sum(e @ v[j * 4:(j + 1) * 4] for j, e in enumerate(e_blocks))
    dense_den = sum(e.sum(axis=1) for e in e_blocks)
    S = np.array([e.sum() for e in e_blocks]); S /= S.sum()
    pi = opl.inclusion_probabilities(S, s)
    num = np.zeros_like(dense_num); den = np.zeros_like(dense_den)
    for g in range(G):
        idx, _, _, _ = opl.sip_row(S, s, (g * UNIT) // G)
        for j in idx:
            num += e_blocks[j] @ v[j * 4:(j + 1) * 4] / pi[j]
            den += e_blocks[j].sum(axis=1) / pi[j]
    bn = sum(np.abs(e_blocks[j] @ v[j * 4:(j + 1) * 4]) / pi[j] for j in range(M)) / G
    bd = sum(e_blocks[j].sum(axis=1) / pi[j] for j in range(M)) / G
    assert np.all(np.abs(num / G - dense_num) <= bn + 1e-9)
    assert np.all(np.abs(den / G - dense_den) <= bd + 1e-9)


def test_keys_beyond_nk_are_masked():
    q, k, v = _head(1, 10, 13, 32, seed=6)       # N = 130: last 4-block has 2 rows
    N = q.shape[0]
    M = -(-N // 4)
    idx = np.tile(np.arange(M), (2, 1))
    O, _ = oat.attn_fwd(q, k, v, 128, 4, idx, None, np.full(2, M))
    ref, _ = oat.dense_attn(q, k, v)
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)


def test_topk_plan_attention_equals_dense_over_selected_keys():
    q, k, v = _head(1, 8, 16, 32, seed=7)
    S = np.random.default_rng(1).random((1, 32))
    idx, bias, cnt, _ = opl.plan(S, 5, opl.TOPK)
    O, _ = oat.attn_fwd(q, k, v, 128, 4, idx, bias, cnt)
    keys = np.concatenate([np.arange(j * 4, j * 4 + 4) for j in idx[0]])
    ref, _ = oat.dense_attn(q, k[keys], v[keys])
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)


def _sdpa_over(q, k, v, keys, shift):
    """torch fp64 SDPA over the given key rows with an additive per-key shift."""
    tq = torch.from_numpy(q)[None, None]
    tk = torch.from_numpy(k[keys])[None, None]
    tv = torch.from_numpy(v[keys])[None, None]
    mask = torch.from_numpy(np.broadcast_to(shift, (q.shape[0], len(keys))).copy())[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)[0, 0].numpy()


def test_list_entries_outside_range_and_count_clamping():
    """The list rules of the boundary: entries outside [0, M) (-1, M, 2^30 + 1,
    -2^31) name no block and are skipped, a block listed twice counts twice,
    the count is clamped to [0, L] (negative -> empty, beyond L -> L), and an
    empty row gives zeros with LSE -inf.  Checked against torch SDPA over the
    explicitly listed key rows (Nk = 130: block 32 holds 2 keys)."""
    q, k, v = _head(1, 10, 39, 32, seed=8)       # Nq = 390: 4 query blocks (last 6 rows)
    k, v = k[:130], v[:130]
    M = 33
    L = 8
    idx = np.full((4, L), 5, np.int64)
    bias = np.random.default_rng(2).random((4, L)).astype(np.float32)
    idx[0] = [3, -1, M, 2**30 + 1, -2**31, 32, 3, 0]
    idx[1] = [1, 2, 3, 4, 5, 6, 7, 8]
    idx[2] = [-1, M, 40, -7, 9, 9, 9, 9]
    idx[3] = [10, 11, 12, 13, 14, 15, 16, 17]
    cnt = np.array([8, -1, 5, 99])
    O, lse = oat.attn_fwd(q, k, v, 128, 4, idx, bias, cnt)
    # row 0: entries 0, 5, 6, 7 are blocks 3, 32, 3, 0
    keep = [(3, 0), (32, 5), (3, 6), (0, 7)]
    keys = np.concatenate([np.arange(j * 4, min(130, j * 4 + 4)) for j, _ in keep])
    shift = np.concatenate([np.full(min(130, j * 4 + 4) - j * 4, np.float64(bias[0, e]))
                            for j, e in keep])
    np.testing.assert_allclose(O[:128], _sdpa_over(q[:128], k, v, keys, shift),
                               rtol=1e-10, atol=1e-12)
    # row 1: count -1 -> no key; row 2: the first five entries, only block 9 valid
    assert np.all(O[128:256] == 0) and np.all(np.isneginf(lse[128:256]))
    keys = np.arange(36, 40)
    np.testing.assert_allclose(O[256:384], _sdpa_over(q[256:384], k, v, keys,
                                                      np.full(4, np.float64(bias[2, 4]))),
                               rtol=1e-10, atol=1e-12)
    # row 3: count beyond L -> all L entries
    keys = np.arange(40, 72)
    shift = np.repeat(bias[3].astype(np.float64), 4)
    np.testing.assert_allclose(O[384:], _sdpa_over(q[384:], k, v, keys, shift),
                               rtol=1e-10, atol=1e-12)
    # the backward skips by the same rule: its dq of the empty row is zero
    dq, _, _ = oat.attn_bwd(q, k, v, np.ones_like(q), 128, 4, idx, bias, cnt)
    assert np.all(dq[128:256] == 0)


def test_list_row_of_only_invalid_entries_is_empty():
    q, k, v = _head(1, 8, 16, 32, seed=9)
    idx = np.array([[-1, -1, 32, 99]])
    O, lse = oat.attn_fwd(q, k, v, 128, 4, idx, None, [4])
    assert np.all(O == 0) and np.all(np.isneginf(lse))
    O, lse = oat.attn_fwd(q, k, v, 128, 4, idx, None, [0])
    assert np.all(O == 0) and np.all(np.isneginf(lse))
