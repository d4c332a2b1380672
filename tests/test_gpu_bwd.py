"""GPU parity of bsa_attn_bwd and bsa_attn_bwd_ws against the fp64 oracle
(oracle/attn.py: attn_bwd) on plans built by the oracle.  The device gets the oracle's
forward output rounded to bf16 and its log-sum-exp rounded to fp32 (the
inputs the forward kernel would hand over); the oracle keeps its exact
values.

Tolerance (per tensor, over the rows checked): relative Frobenius error
<= 1e-2 and max-abs error <= 2e-2 of the tensor's largest magnitude.  The
device rounds P and dS to bf16 before the two products that use them (a
random relative error of 2^-9 per term, averaged over the contraction),
takes D = dO . O from the bf16 forward output, and sums in fp32; dK and dV
add contributions of many query blocks with fp32 atomics (bsa_attn_bwd) or
sum per-entry partial rows in fp32 (bsa_attn_bwd_ws)."""
import numpy as np
import pytest

from oracle import attn as oat
from oracle import plan as opl
from oracle import select as osel
from synth import CONFIGS, bf16_bits_to_f64, f64_to_bf16_bits, make_qkv

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2
MAX_ABS_FRAC = 2e-2
VARIANTS = ("atomic", "ws")


def _bwd(bsa, variant, *args, slabs=None, **kw):
    """One backward call through the atomic or the workspace entry point."""
    if variant == "atomic":
        return bsa.bsa_attn_bwd(*args, **kw)
    return bsa.bsa_attn_bwd_ws(*args, slabs=slabs, **kw)


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def _plan(nqb, M, s, mode, seed):
    rng = np.random.default_rng(seed)
    S = rng.gamma(0.4, size=(nqb, M))
    S /= S.sum(axis=1, keepdims=True)
    return opl.plan(S, s, mode, seed=seed)


def _close(g, got, want, what, rows=None):
    if rows is not None:
        got, want = got[rows], want[rows]
    err = np.abs(got - want)
    fro = float(np.sqrt((err ** 2).sum() / max((want ** 2).sum(), 1e-300)))
    mx = float(err.max() / max(np.abs(want).max(), 1e-300))
    g.say(f"  {what}: rel fro {fro:.2e}, max-abs/max {mx:.2e}")
    assert fro <= REL_FRO, f"{what}: relative Frobenius error {fro}"
    assert mx <= MAX_ABS_FRAC, f"{what}: max-abs error {mx} of the largest magnitude"


def _oracle_fwd(q, k, v, kvb, idx, bias, cnt):
    """The oracle's forward; a query block with an empty (valid) list gets
    output 0 and lse -inf, as the forward kernel documents."""
    live = [i for i in range(idx.shape[0]) if cnt[i] > 0]
    O, lse = oat.attn_fwd(q, k, v, 128, kvb, idx, bias, cnt, blocks=live)
    return np.nan_to_num(O), np.where(np.isnan(lse), -np.inf, lse)


def _run(env, variant, q, k, v, dout, kvb, idx, bias, cnt):
    """Device backward of one head (B = H = 1) with the oracle's forward
    (valid list entries only)."""
    bsa, g, torch = env
    O, lse = _oracle_fwd(q, k, v, kvb, idx, bias, cnt)
    ob = f64_to_bf16_bits(O)
    dev = lambda x: g.to_dev_bf16(f64_to_bf16_bits(x)[None, None])  # noqa: E731
    dq, dk, dv = _bwd(bsa, variant, dev(q), dev(k), dev(v), g.to_dev_bf16(ob[None, None]),
                      dev(dout), g.dev_f32(lse[None, None]), g.dev_i32(idx[None, None]),
                      None if bias is None else g.dev_f32(bias[None, None]),
                      g.dev_i32(cnt[None, None]), 128, kvb)
    torch.cuda.synchronize()
    return dq.cpu().numpy()[0, 0], dk.cpu().numpy()[0, 0], dv.cpu().numpy()[0, 0]


def _inputs(Nq, Nk, seed, d=128):
    qb, _, _ = make_qkv(1, 1, Nq, 1, d, seed=seed)
    _, kb, vb = make_qkv(1, 1, Nk, 1, d, seed=seed + 1)
    db, _, _ = make_qkv(1, 1, Nq, 1, d, seed=seed + 2)
    return tuple(bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb, db))


@pytest.mark.parametrize("Nq,Nk,kvb,s,mode,d", [
    (300, 300, 4, 20, opl.SIP, 128), (256, 256, 1, 60, opl.SIP, 128),
    (512, 512, 16, 9, opl.TOPK, 128), (1000, 1000, 128, 3, opl.SIP, 128),
    (384, 390, 8, 30, opl.SIP, 128), (200, 700, 4, 50, opl.TOPK, 128),
    (130, 2048, 2, 600, opl.SIP, 128),
    (300, 300, 4, 20, opl.SIP, 64), (256, 260, 1, 70, opl.SIP, 64), (640, 2048, 64, 8, opl.TOPK, 64),
    (130, 2048, 2, 600, opl.SIP, 64),
    (256, 5000, 1, 4500, opl.SIP, 128),
])
@pytest.mark.parametrize("variant", VARIANTS)
def test_bwd_matches_oracle(env, variant, Nq, Nk, kvb, s, mode, d):
    """Ragged query and key counts (a partial last KV block), block sizes 1-128,
    SIP shifts and top-k, lists longer than one staging phase, d = 64 and 128,
    and lists of 4,500 entries (past the 4,096 the workspace form's pair
    union searches in LDS, so that pair takes the concatenated union)."""
    bsa, g, torch = env
    g.say(f"case bwd {variant} Nq={Nq} Nk={Nk} kv={kvb} s={s} mode={mode} d={d}")
    q, k, v, dout = _inputs(Nq, Nk, seed=Nq + kvb, d=d)
    nqb, M = -(-Nq // 128), -(-Nk // kvb)
    idx, bias, cnt, _ = _plan(nqb, M, s, mode, seed=Nk)
    gq, gk, gv = _run(env, variant, q, k, v, dout, kvb, idx, bias if mode == opl.SIP else None,
                      cnt)
    wq, wk, wv = oat.attn_bwd(q, k, v, dout, 128, kvb, idx, bias if mode == opl.SIP else None, cnt)
    _close(g, gq, wq, "dq")
    _close(g, gk, wk, "dk")
    _close(g, gv, wv, "dv")


@pytest.mark.parametrize("variant", VARIANTS)
def test_bwd_edge_lists(env, variant):
    """Invalid entries (negative, past M), a repeated block (two sets of keys),
    an empty list, count beyond the list and a block holding keys past Nk:
    the device on the raw list against the oracle, whose forward (for the
    device's inputs) runs on the list's valid entries.  dk and dv start as
    NaN: every row, listed or not, must be written."""
    bsa, g, torch = env
    g.say(f"case bwd {variant} edge lists")
    Nq, Nk, kvb = 384, 257, 4
    q, k, v, dout = _inputs(Nq, Nk, seed=5)
    M = -(-Nk // kvb)
    assert M == 65
    idx = np.array([[3, -1, 70, 3, 64, 10, 11, 12],
                    [0, 1, 2, 3, 4, 5, 6, 7],
                    [9, 9, 9, 20, 30, 40, 64, 1]], np.int32)
    bias = np.random.default_rng(1).random(idx.shape).astype(np.float32)
    cnt = np.array([8, 0, 20], np.int32)
    ci = np.full((3, 8), -1, np.int32)
    cb = np.zeros((3, 8), np.float32)
    cc = np.zeros(3, np.int32)
    for i in range(3):
        keep = [e for e in range(min(int(cnt[i]), 8)) if 0 <= idx[i, e] < M]
        ci[i, :len(keep)], cb[i, :len(keep)], cc[i] = idx[i, keep], bias[i, keep], len(keep)
    O, lse = _oracle_fwd(q, k, v, kvb, ci, cb, cc)
    dev = lambda x: g.to_dev_bf16(f64_to_bf16_bits(x)[None, None])  # noqa: E731
    nan = torch.full((1, 1, Nk, 128), float("nan"), dtype=torch.float32, device="cuda")
    gq, gk, gv = _bwd(bsa, variant, dev(q), dev(k), dev(v), dev(O), dev(dout),
                      g.dev_f32(lse[None, None]), g.dev_i32(idx[None, None]),
                      g.dev_f32(bias[None, None]), g.dev_i32(cnt[None, None]), 128, kvb,
                      dk=nan.clone(), dv=nan.clone())
    torch.cuda.synchronize()
    gq, gk, gv = (x.cpu().numpy()[0, 0] for x in (gq, gk, gv))
    wq, wk, wv = oat.attn_bwd(q, k, v, dout, 128, kvb, idx, bias, cnt)
    _close(g, gq, wq, "dq (listed blocks)", np.r_[0:128, 256:384])
    assert not gq[128:256].any()           # empty list: zero gradient
    _close(g, gk, wk, "dk")
    _close(g, gv, wv, "dv")


@pytest.mark.parametrize("kvb", [4, 1, 128])
@pytest.mark.parametrize("variant", VARIANTS)
def test_bwd_pair_classes(env, variant, kvb):
    """The workspace form runs query blocks (2m, 2m + 1) together over the
    union of their lists, grouped into blocks both list, the first only and
    the second only.  Pairs built for each case: identical blocks with
    different shifts (all shared), disjoint lists (none shared), lists that
    share a part, a list in descending order and one with a repeated block
    (both not ascending: the pair falls back to one list after the other),
    an empty list beside a full one, and a last query block of 40 rows
    alone in its pair.  KV blocks of 4 (32 blocks per 128-key pass), 1 (128)
    and 128 (one)."""
    bsa, g, torch = env
    g.say(f"case bwd {variant} pair classes kv={kvb}")
    Nq, Nk, s = 10 * 128 + 40, 1500, 40
    nqb, M = -(-Nq // 128), -(-Nk // kvb)
    s = min(s, M // 2)
    q, k, v, dout = _inputs(Nq, Nk, seed=40 + kvb)
    rng = np.random.default_rng(kvb)
    idx = np.full((nqb, s), -1, np.int32)
    cnt = np.full(nqb, s, np.int32)
    perm = rng.permutation(M)
    a, b = np.sort(perm[:s]), np.sort(perm[s:2 * s])
    idx[0], idx[1] = a, a                                # all shared
    idx[2], idx[3] = a, b                                # none shared
    idx[4], idx[5] = a, np.sort(np.concatenate([a[: s // 2], b[: s - s // 2]]))  # half shared
    idx[6], idx[7] = a[::-1], a                          # descending: fallback
    idx[8] = a
    idx[8, 1] = a[0]                                     # repeated block: fallback
    idx[9], cnt[9] = b, 0                                # empty beside the pair's other
    idx[10] = np.sort(rng.choice(M, s, replace=False))   # 40 rows, a pair of one
    bias = rng.random(idx.shape).astype(np.float32) * 3.0
    gq, gk, gv = _run(env, variant, q, k, v, dout, kvb, idx, bias, cnt)
    wq, wk, wv = oat.attn_bwd(q, k, v, dout, 128, kvb, idx, bias, cnt)
    _close(g, gq[: 9 * 128], wq[: 9 * 128], "dq")
    assert not gq[9 * 128: 10 * 128].any()               # empty list: zero gradient
    _close(g, gq[10 * 128:], wq[10 * 128:], "dq last block")
    _close(g, gk, wk, "dk")
    _close(g, gv, wv, "dv")


def test_bwd_ws_deterministic(env):
    """The workspace form sums each KV block's partial rows in ascending slot
    order, so dK and dV are the same bits on every call and for any number
    of slabs per pass (B = 1, H = 3: all slabs in one pass, then one per
    pass)."""
    bsa, g, torch = env
    g.say("case bwd ws deterministic")
    H, N, kvb, s = 3, 1000, 4, 60
    nqb, M = -(-N // 128), N // 4
    qs, ks, vs, ds, Os, ls, ids, bs, cs = ([] for _ in range(9))
    for h in range(H):
        q, k, v, dout = _inputs(N, N, seed=200 + h)
        idx, bias, cnt, _ = _plan(nqb, M, s, opl.SIP, seed=h)
        O, lse = _oracle_fwd(q, k, v, kvb, idx, bias, cnt)
        for lst, x in zip((qs, ks, vs, ds, Os, ls, ids, bs, cs),
                          (q, k, v, dout, O, lse, idx, bias, cnt)):
            lst.append(x)
    st = lambda xs: np.stack(xs)[None]  # noqa: E731
    bf = lambda xs: g.to_dev_bf16(f64_to_bf16_bits(st(xs)))  # noqa: E731
    args = (bf(qs), bf(ks), bf(vs), bf(Os), bf(ds), g.dev_f32(st(ls)), g.dev_i32(st(ids)),
            g.dev_f32(st(bs)), g.dev_i32(st(cs)), 128, kvb)
    runs = [bsa.bsa_attn_bwd_ws(*args, slabs=n) for n in (None, None, 1)]
    torch.cuda.synchronize()
    for r, run in enumerate(runs[1:], 1):
        for name, a_, b_ in zip(("dq", "dk", "dv"), runs[0], run):
            assert torch.equal(a_, b_), f"call {r}: {name} differs"
    wq, wk, wv = oat.attn_bwd(qs[0], ks[0], vs[0], ds[0], 128, kvb, ids[0], bs[0], cs[0])
    _close(g, runs[0][1].cpu().numpy()[0, 0], wk, "h0 dk")


@pytest.mark.parametrize("variant,slabs", [("atomic", None), ("ws", None), ("ws", 1), ("ws", 3)])
def test_bwd_batch_heads(env, variant, slabs):
    """B = 2, H = 2 in one call: every (b, h) against the oracle.  The
    workspace variant also runs with room for one slab (four passes) and
    for three (a pass of three, then one)."""
    bsa, g, torch = env
    g.say(f"case bwd {variant} slabs={slabs} batch and heads")
    B, H, N, kvb, s = 2, 2, 400, 4, 25
    nqb, M = -(-N // 128), N // 4
    qs, ks, vs, ds, Os, ls, ids, bs, cs = ([] for _ in range(9))
    for b in range(B):
        for h in range(H):
            q, k, v, dout = _inputs(N, N, seed=100 + 10 * b + h)
            idx, bias, cnt, _ = _plan(nqb, M, s, opl.SIP, seed=b * H + h)
            O, lse = _oracle_fwd(q, k, v, kvb, idx, bias, cnt)
            for lst, x in zip((qs, ks, vs, ds, Os, ls, ids, bs, cs),
                              (q, k, v, dout, O, lse, idx, bias, cnt)):
                lst.append(x)
    st = lambda xs: np.stack(xs).reshape((B, H) + xs[0].shape)  # noqa: E731
    bf = lambda xs: g.to_dev_bf16(f64_to_bf16_bits(st(xs)))  # noqa: E731
    dq, dk, dv = _bwd(bsa, variant, bf(qs), bf(ks), bf(vs), bf(Os), bf(ds), g.dev_f32(st(ls)),
                      g.dev_i32(st(ids)), g.dev_f32(st(bs)), g.dev_i32(st(cs)), 128, kvb,
                      slabs=slabs)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            j = b * H + h
            wq, wk, wv = oat.attn_bwd(qs[j], ks[j], vs[j], ds[j], 128, kvb, ids[j], bs[j], cs[j])
            _close(g, dq.cpu().numpy()[b, h], wq, f"b{b} h{h} dq")
            _close(g, dk.cpu().numpy()[b, h], wk, f"b{b} h{h} dk")
            _close(g, dv.cpu().numpy()[b, h], wv, f"b{b} h{h} dv")


@pytest.mark.parametrize("workload", ["wan14b_720p", "hunyuan_720p"])
def test_bwd_full_size_sampled(env, workload):
    """Wan2.1-14B 720p shape (SIP budget 2048 of 18,900 4-token blocks) and
    HunyuanVideo 720p shape (2272 of 29,700), one head, the oracle's SIP
    plan: the device forward's output and LSE feed the device backward; dQ
    of sampled query blocks (including the ragged last: 80 and 16 rows) and
    dK/dV of sampled KV blocks (all query blocks that list them) against the
    oracle.  The workspace variant against the oracle on the same samples,
    and against the atomic one on every row: dq bit for bit (the same
    kernel), dk and dv to fp32 summation-order error."""
    bsa, g, torch = env
    c = CONFIGS[workload]
    g.say(f"case bwd full size {workload} head 0")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    db, _, _ = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=77)
    S, _, _ = osel.select_scores_head(qb[0, 0], kb[0, 0], 128, 4, 8, 1)
    idx, bias, cnt, _ = opl.plan(S, c["budget"], opl.SIP, seed=0)
    q, k, v, dq_, = (g.to_dev_bf16(x) for x in (qb, kb, vb, db))
    di, dbias, dc = g.dev_i32(idx[None, None]), g.dev_f32(bias[None, None]), g.dev_i32(cnt[None, None])
    out, lse = bsa.bsa_attn_fwd(q, k, v, di, dbias, dc, 128, 4, want_lse=True)
    gq, gk, gv = bsa.bsa_attn_bwd(q, k, v, out, dq_, lse, di, dbias, dc, 128, 4)
    g.say("  workspace variant")
    sq, sk, sv = bsa.bsa_attn_bwd_ws(q, k, v, out, dq_, lse, di, dbias, dc, 128, 4)
    torch.cuda.synchronize()
    gq, gk, gv, sq, sk, sv = (x.cpu().numpy()[0, 0] for x in (gq, gk, gv, sq, sk, sv))
    assert np.array_equal(gq, sq)
    for a_, b_, what in ((gk, sk, "dk"), (gv, sv, "dv")):
        fro = float(np.sqrt(((a_.astype(np.float64) - b_) ** 2).sum() / (a_.astype(np.float64) ** 2).sum()))
        g.say(f"  {what} workspace vs atomic: rel fro {fro:.2e}")
        assert fro <= 1e-5, f"{what}: workspace and atomic variants differ by {fro}"
    q64, k64, v64, d64 = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb, db))
    nqb = idx.shape[0]
    qblocks = [0, 1, 300, nqb - 1]
    wq, _, _ = oat.attn_bwd(q64, k64, v64, d64, 128, 4, idx, bias, cnt, blocks=qblocks)
    rows = np.concatenate([np.arange(i * 128, min(q64.shape[0], i * 128 + 128)) for i in qblocks])
    _close(g, gq, wq, "dq sampled query blocks", rows)
    kvblocks = [int(idx[0, 0]), int(idx[300, 1000]), int(idx[nqb - 1, -1])]
    users = sorted({i for i in range(nqb) if np.isin(kvblocks, idx[i, :cnt[i]]).any()})
    g.say(f"  {len(users)} query blocks list the sampled KV blocks {kvblocks}")
    _, wk, wv = oat.attn_bwd(q64, k64, v64, d64, 128, 4, idx, bias, cnt, blocks=users)
    krows = np.concatenate([np.arange(j * 4, j * 4 + 4) for j in kvblocks])
    _close(g, gk, wk, "dk sampled KV blocks", krows)
    _close(g, gv, wv, "dv sampled KV blocks", krows)
    _close(g, sk, wk, "dk (workspace) sampled KV blocks", krows)
    _close(g, sv, wv, "dv (workspace) sampled KV blocks", krows)
