"""GPU parity of bsa_attn_fwd against the fp64 oracle (plain masked, shifted
softmax over the gathered keys), on plans built by the oracle so that this
check does not depend on the selector or the planner."""
import numpy as np
import pytest

from oracle import attn as oat
from oracle import plan as opl
from oracle import select as osel
from synth import CONFIGS, bf16_bits_to_f64, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def _random_plan(nqb, M, s, mode, seed, zeros=0):
    rng = np.random.default_rng(seed)
    S = rng.gamma(0.4, size=(nqb, M))
    if zeros:
        S[:, rng.integers(0, M, zeros)] = 0.0
    S /= S.sum(axis=1, keepdims=True)
    return opl.plan(S, s, mode, seed=seed)


def _run(env, qb, kb, vb, kvb, idx, bias, cnt, Nq=None, want_lse=True):
    bsa, g, torch = env
    q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    B, H, _, d = q.shape
    nqb = idx.shape[2]
    out, lse = bsa.bsa_attn_fwd(q, k, v, g.dev_i32(idx), None if bias is None else g.dev_f32(bias),
                                g.dev_i32(cnt), 128, kvb, want_lse=want_lse)
    torch.cuda.synchronize()
    return g.from_dev_bf16(out), (lse.cpu().numpy() if lse is not None else None)


@pytest.mark.parametrize("N,d,kvb,mode", [
    (128, 64, 4, opl.SIP), (256, 128, 1, opl.SIP), (512, 128, 16, opl.TOPK),
    (1000, 128, 4, opl.SIP), (1000, 64, 64, opl.TOPK), (640, 128, 128, opl.SIP),
    (896, 128, 2, opl.SIP), (384, 64, 8, opl.SIP),
])
def test_attn_matches_oracle_fuzz(env, N, d, kvb, mode):
    bsa, g, torch = env
    g.say(f"case attn fuzz N={N} d={d} kv_block={kvb} mode={mode}")
    qb, kb, vb = make_qkv(1, 1, N, 2, d, seed=N + d + kvb)
    M = -(-N // kvb)
    nqb = -(-N // 128)
    s = max(1, M // 5)
    idx = np.zeros((1, 2, nqb, s), np.int32)
    bias = np.zeros((1, 2, nqb, s), np.float32)
    cnt = np.zeros((1, 2, nqb), np.int32)
    for h in range(2):
        i_, b_, c_, _ = _random_plan(nqb, M, s, mode, seed=h + N)
        idx[0, h], bias[0, h], cnt[0, h] = i_, b_, c_
    O, lse = _run(env, qb, kb, vb, kvb, idx, bias, cnt)
    for h in range(2):
        q, k, v = (bf16_bits_to_f64(x[0, h]) for x in (qb, kb, vb))
        ref, rlse = oat.attn_fwd(q, k, v, 128, kvb, idx[0, h], bias[0, h], cnt[0, h])
        g.assert_attn_close(O[0, h], ref, f"head {h}")
        np.testing.assert_allclose(lse[0, h], rlse, rtol=0, atol=2e-3)


def test_attn_tiny_topk_config(env):
    """Tiny grid 2x32x32, d = 64, KV block 64, mean-pooled scores (one
    cluster), top-8 per query block, pi = 1; every query row checked."""
    bsa, g, torch = env
    c = CONFIGS["tiny_2x32x32"]
    g.say("case attn tiny 2x32x32 top-8")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    S, _, _ = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, c["kv_block"], 1, 1)
    idx, bias, cnt, _ = opl.plan(S, c["budget"], opl.TOPK)
    O, _ = _run(env, qb, kb, vb, c["kv_block"], idx[None, None], None, cnt[None, None])
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    ref, _ = oat.attn_fwd(q, k, v, 128, c["kv_block"], idx, None, cnt)
    g.assert_attn_close(O[0, 0], ref, "tiny")


def test_attn_all_blocks_equals_dense(env):
    bsa, g, torch = env
    g.say("case attn dense equivalence N=768 d=128")
    qb, kb, vb = make_qkv(1, 24, 32, 1, 128, seed=3)
    N = 768
    M = N // 4
    idx = np.tile(np.arange(M, dtype=np.int32), (1, 1, 6, 1))
    cnt = np.full((1, 1, 6), M, np.int32)
    O, _ = _run(env, qb, kb, vb, 4, idx, None, cnt)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    ref, _ = oat.dense_attn(q, k, v)
    g.assert_attn_close(O[0, 0], ref, "dense")


def test_attn_edge_rows(env):
    """count 0 -> zeros and lse -inf; out-of-range indices are skipped;
    entries beyond count are ignored; Nk smaller than Nq."""
    bsa, g, torch = env
    g.say("case attn edge rows")
    qb, kb, vb = make_qkv(1, 1, 384, 1, 64, seed=5)
    kb2, vb2 = kb[:, :, :130], vb[:, :, :130]           # Nk = 130: last 4-block has 2 rows
    M = 33
    idx = np.full((1, 1, 3, 12), 7, np.int32)
    cnt = np.array([[[0, 12, 9]]], np.int32)
    idx[0, 0, 1] = [0, 5, -1, 32, 40, 2, 3, 1000, 4, 6, 8, 9]
    idx[0, 0, 2, :9] = [32, 31, 30, 0, 1, 2, 3, 4, 5]
    bias = np.random.default_rng(0).random((1, 1, 3, 12)).astype(np.float32)
    O, lse = _run(env, qb, kb2, vb2, 4, idx, bias, cnt)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb2, vb2))
    assert np.all(O[0, 0, :128] == 0) and np.all(np.isneginf(lse[0, 0, :128]))
    ref1, _ = oat.attn_fwd(q[128:256], k, v, 128, 4, idx[0, 0, 1][None], bias[0, 0, 1][None],
                           [12])
    g.assert_attn_close(O[0, 0, 128:256], ref1, "row with invalid indices")
    ref2, _ = oat.attn_fwd(q[256:], k, v, 128, 4, idx[0, 0, 2][None], bias[0, 0, 2][None], [9])
    g.assert_attn_close(O[0, 0, 256:], ref2, "row with partial block")


@pytest.mark.parametrize("d,Nk,kvb", [(128, 260, 2), (128, 130, 2), (128, 6, 2), (128, 131, 2),
                                      (64, 136, 4), (64, 132, 4), (64, 4, 4),
                                      (128, 132, 8), (128, 260, 4), (64, 136, 16),
                                      (128, 130, 4), (128, 263, 8), (128, 3, 4), (64, 131, 8),
                                      (64, 5, 16)])
def test_attn_group_shift_edges(env, d, Nk, kvb):
    """The group-shift path (every wave load inside one KV block): a row with
    count 0, invalid indices (-1, M, 1000, and 2^30 + 1 and -2^31, whose key
    row wraps around in 32-bit arithmetic) among valid ones, entries past the
    count, and the partial last block -- whole groups past Nk, and (Nk not a
    whole number of wave loads) a load and a 4-key group crossing Nk, down
    to Nk smaller than one load.  KV blocks of half a wave load (2 tokens at
    d = 128, 4 at d = 64) take the half-load variant of the path when Nk is
    a whole number of blocks (Nk = 131 at 2-token blocks takes the per-key
    path)."""
    bsa, g, torch = env
    g.say(f"case attn group-shift edges d={d} Nk={Nk} kv_block={kvb}")
    qb, kb, vb = make_qkv(1, 1, 384, 1, d, seed=Nk + kvb)
    kb2, vb2 = kb[:, :, :Nk], vb[:, :, :Nk]
    M = -(-Nk // kvb)
    idx = np.full((1, 1, 3, 14), M + 5, np.int32)
    cnt = np.array([[[0, 14, 9]]], np.int32)
    idx[0, 0, 1] = [0, 5 % M, -1, M - 1, M, 2, 3, 1000, 4 % M, 1, M - 2, 6 % M, 2**30 + 1, -2**31]
    idx[0, 0, 2, :9] = [M - 1, M - 2, 0, 1, 2, 3, 4 % M, 5 % M, 6 % M]
    bias = np.random.default_rng(1).random((1, 1, 3, 14)).astype(np.float32)
    O, lse = _run(env, qb, kb2, vb2, kvb, idx, bias, cnt)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb2, vb2))
    assert np.all(O[0, 0, :128] == 0) and np.all(np.isneginf(lse[0, 0, :128]))
    for i in (1, 2):
        ref, rlse = oat.attn_fwd(q[128 * i:128 * i + 128], k, v, 128, kvb, idx[0, 0, i][None],
                                 bias[0, 0, i][None], [cnt[0, 0, i]])
        g.assert_attn_close(O[0, 0, 128 * i:128 * i + 128], ref, f"row {i}")
        np.testing.assert_allclose(lse[0, 0, 128 * i:128 * i + 128], rlse, rtol=0, atol=2e-3)


def test_attn_multi_phase_lists(env):
    """Lists longer than one staging phase (4096 keys of group shifts; 512
    entries of per-key shifts), with ragged counts: exactly one phase, one
    entry more, a ragged second phase, and the full list; sampled query
    blocks against the oracle, for both shift paths (Nk a multiple of 4 or
    not)."""
    bsa, g, torch = env
    for N in (12000, 11999):
        g.say(f"case attn multi-phase N={N} d=128 kv_block=4")
        qb, kb, vb = make_qkv(1, 1, N, 1, 128, seed=N)
        M = -(-N // 4)
        nqb = -(-N // 128)
        s = 1500
        i_, b_, c_, _ = _random_plan(nqb, M, s, opl.SIP, seed=N)
        c_ = c_.copy()
        c_[0], c_[1], c_[2], c_[3] = 1024, 1025, 1200, 511
        O, _ = _run(env, qb, kb, vb, 4, i_[None, None], b_[None, None], c_[None, None],
                    want_lse=False)
        q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
        blocks = [0, 1, 2, 3, 40, nqb - 1]
        ref, _ = oat.attn_fwd(q, k, v, 128, 4, i_, b_, c_, blocks=blocks)
        rows = np.concatenate([np.arange(i * 128, min(N, i * 128 + 128)) for i in blocks])
        g.assert_attn_close(O[0, 0][rows], ref[rows], f"N={N} sampled blocks")


@pytest.mark.parametrize("d,kvb,N", [(128, 2, 12000), (128, 2, 11999), (64, 4, 12000)])
def test_attn_multi_phase_half_loads(env, d, kvb, N):
    """KV blocks of half a wave load with lists longer than one staging phase
    (1,024 entries): exactly one phase, one entry more, a ragged third phase
    and a short list; N = 11,999 (a partial last block) takes the per-key
    path instead."""
    bsa, g, torch = env
    g.say(f"case attn multi-phase half loads N={N} d={d} kv_block={kvb}")
    qb, kb, vb = make_qkv(1, 1, N, 1, d, seed=N + d)
    M = -(-N // kvb)
    nqb = -(-N // 128)
    s = 3000
    i_, b_, c_, _ = _random_plan(nqb, M, s, opl.SIP, seed=N + kvb)
    c_ = c_.copy()
    c_[0], c_[1], c_[2], c_[3] = 1024, 1025, 2500, 511
    O, _ = _run(env, qb, kb, vb, kvb, i_[None, None], b_[None, None], c_[None, None],
                want_lse=False)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    blocks = [0, 1, 2, 3, 40, nqb - 1]
    ref, _ = oat.attn_fwd(q, k, v, 128, kvb, i_, b_, c_, blocks=blocks)
    rows = np.concatenate([np.arange(i * 128, min(N, i * 128 + 128)) for i in blocks])
    g.assert_attn_close(O[0, 0][rows], ref[rows], f"N={N} d={d} kv={kvb} sampled blocks")


def test_attn_fuzz_geometries(env):
    """Random small shapes through both shift paths (group shifts when the KV
    block covers a wave load and Nk is a whole number of loads, per-key
    shifts otherwise): lists with invalid entries, repeated blocks, counts
    from 0 to the list length, shifts from 0 to 8."""
    bsa, g, torch = env
    rng = np.random.default_rng(2024)
    for case in range(24):
        d = int(rng.choice([64, 128]))
        kvb = int(rng.choice([1, 2, 4, 8, 16, 32]))
        N = int(rng.integers(1, 400))
        Nk = int(rng.integers(max(1, N // 2), N + 1))
        M = -(-Nk // kvb)
        nqb = -(-N // 128)
        L = int(rng.integers(1, 2 * M + 3))
        g.say(f"case attn fuzz {case}: N={N} Nk={Nk} d={d} kv_block={kvb} list={L}")
        qb, kb, vb = make_qkv(1, 1, N, 1, d, seed=case)
        kb, vb = kb[:, :, :Nk], vb[:, :, :Nk]
        idx = rng.integers(-2, M + 3, (1, 1, nqb, L)).astype(np.int32)
        bias = (rng.random((1, 1, nqb, L)) * 8).astype(np.float32)
        bias[rng.random((1, 1, nqb, L)) < 0.3] = 0.0
        cnt = rng.integers(0, L + 1, (1, 1, nqb)).astype(np.int32)
        O, lse = _run(env, qb, kb, vb, kvb, idx, bias, cnt)
        q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
        ref, rlse = oat.attn_fwd(q, k, v, 128, kvb, idx[0, 0], bias[0, 0], cnt[0, 0])
        for i in range(nqb):
            rows = slice(128 * i, min(N, 128 * i + 128))
            if np.isneginf(rlse[rows]).all():
                assert np.all(O[0, 0, rows] == 0), f"case {case} block {i}: empty list not zero"
                assert np.isneginf(lse[0, 0, rows]).all()
                continue
            g.assert_attn_close(O[0, 0, rows], ref[rows], f"case {case} block {i}")
            np.testing.assert_allclose(lse[0, 0, rows], rlse[rows], rtol=0, atol=2e-3)


def test_attn_deterministic(env):
    bsa, g, torch = env
    g.say("case attn determinism")
    qb, kb, vb = make_qkv(1, 8, 128, 2, 128, seed=9)
    N = 1024
    i_, b_, c_, _ = _random_plan(8, N // 4, 50, opl.SIP, seed=1)
    idx = np.stack([i_, i_])[None]
    bias = np.stack([b_, b_])[None]
    cnt = np.stack([c_, c_])[None]
    O1, l1 = _run(env, qb, kb, vb, 4, idx, bias, cnt)
    O2, l2 = _run(env, qb, kb, vb, 4, idx, bias, cnt)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_attn_wan13b_head_full_size(env):
    """One head of the Wan2.1-1.3B 480p shape (32,760 tokens, KV block 4,
    budget 887) with the oracle's own SIP plan; 24 sampled query blocks
    including the 120-row last block."""
    bsa, g, torch = env
    c = CONFIGS["wan13b_480p"]
    g.say("case attn wan13b one head full size")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    S, _, _ = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, 4, 8, 1)
    idx, bias, cnt, _ = opl.plan(S, c["budget"], opl.SIP, seed=0)
    O, _ = _run(env, qb, kb, vb, 4, idx[None, None], bias[None, None], cnt[None, None],
                want_lse=False)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    rng = np.random.default_rng(0)
    blocks = sorted(set(rng.choice(255, 23, replace=False).tolist()) | {255})
    ref, _ = oat.attn_fwd(q, k, v, 128, 4, idx, bias, cnt, blocks=blocks)
    rows = np.concatenate([np.arange(i * 128, min(q.shape[0], i * 128 + 128)) for i in blocks])
    g.assert_attn_close(O[0, 0][rows], ref[rows], "wan13b sampled blocks")


@pytest.mark.parametrize("kind", ["dense_kv128", "sip_50pct_kv4"])
def test_attn_high_density_full_size(env, kind):
    """The ends of the latency-density curve at the Wan2.1-14B 720p shape
    (one head, 75,600 tokens): the dense plan (every 128-token block, no
    shift) against the oracle's dense attention, and SIP at half of the
    18,900 4-token blocks (the oracle's scores through the device planner,
    checked equal to the oracle's plan) against the oracle on its own plan;
    sampled query blocks including the 80-row last one."""
    bsa, g, torch = env
    c = CONFIGS["wan14b_720p"]
    g.say(f"case attn high density full size {kind}")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    N = q.shape[0]
    blocks = [0, 1, 300, 590]
    rows = np.concatenate([np.arange(i * 128, min(N, i * 128 + 128)) for i in blocks])
    qd, kd, vd = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    if kind == "dense_kv128":
        idx, cnt = bsa.dense_plan(1, 1, N, N, 128)
        out, _ = bsa.bsa_attn_fwd(qd, kd, vd, idx, None, cnt, 128, 128)
        ref = np.full((N, q.shape[1]), np.nan)
        ref[rows] = oat.dense_attn(q[rows], k, v)[0]
    else:
        s = 9450
        S, _, _ = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, 4, 8, 1)
        idx, bias, cnt, _ = bsa.bsa_sip_plan(g.dev_f32(S[None, None]), s, bsa.PLAN_SIP, seed=0)
        wi, wb, wc, _ = opl.plan(S[blocks], s, opl.SIP,
                                 offsets=[opl.sampling_offset(0, i) for i in blocks])
        np.testing.assert_array_equal(idx[0, 0, blocks].cpu().numpy(), wi)
        np.testing.assert_array_equal(cnt[0, 0, blocks].cpu().numpy(), wc)
        out, _ = bsa.bsa_attn_fwd(qd, kd, vd, idx, bias, cnt, 128, 4)
        fi = np.full((591, s), -1, np.int32)
        fb = np.zeros((591, s), np.float32)
        fc = np.zeros(591, np.int32)
        fi[blocks], fb[blocks], fc[blocks] = wi, wb, wc
        ref, _ = oat.attn_fwd(q, k, v, 128, 4, fi, fb, fc, blocks=blocks)
    torch.cuda.synchronize()
    got = g.from_dev_bf16(out)[0, 0]
    g.assert_attn_close(got[rows], ref[rows], f"{kind} sampled blocks")


def test_attn_hunyuan_head_full_size_topk(env):
    """One head of the HunyuanVideo 720p shape (33 x 45 x 80 = 118,800 tokens,
    KV block 4, budget 2272 of 29,700 blocks) with the oracle's top-k plan on
    the oracle's scores; sampled query blocks including the 16-row last one."""
    bsa, g, torch = env
    c = CONFIGS["hunyuan_720p"]
    g.say("case attn hunyuan one head full size top-k")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    S, _, _ = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, 4, 8, 1)
    idx, bias, cnt, _ = opl.plan(S, c["budget"], opl.TOPK)
    O, _ = _run(env, qb, kb, vb, 4, idx[None, None], None, cnt[None, None], want_lse=False)
    q, k, v = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    nqb = idx.shape[0]
    assert nqb == 929 and q.shape[0] - 128 * (nqb - 1) == 16
    blocks = [0, 464, nqb - 2, nqb - 1]
    ref, _ = oat.attn_fwd(q, k, v, 128, 4, idx, None, cnt, blocks=blocks)
    rows = np.concatenate([np.arange(i * 128, min(q.shape[0], i * 128 + 128)) for i in blocks])
    g.assert_attn_close(O[0, 0][rows], ref[rows], "hunyuan top-k sampled blocks")
