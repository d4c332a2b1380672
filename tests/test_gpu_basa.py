"""GPU parity of the BASA path (bsa_basa_plan -> bsa_attn_fwd ->
bsa_window_unpermute) against the definition-based oracle (oracle/basa.py),
which builds no lists: windows of the rolled grid, routed windows and the
pooled memory are gathered directly and attended in fp64.

Bit-exact: routes (fp32 routing in the stated order on both sides), the
window-major copies of Q/K/V and their zero pad rows, the block lists.
Pooled K/V rows: the device stores the fp32 cell mean rounded to bf16; they
are checked against the oracle's fp64 cell mean within one bf16 step.
Attention output: within the attention tolerances."""
import numpy as np
import pytest

from oracle import basa as obasa
from synth import CONFIGS, bf16_bits_to_f32, bf16_bits_to_f64, make_qkv
from tests import _pool

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def _window_rows(T, Hg, Wg, wh, ww):
    """(first padded row, token count) of every window, window-major order."""
    nwy, nwx = obasa.window_grid(Hg, Wg, wh, ww)
    out, off = [], 0
    for a in range(nwy):
        for b in range(nwx):
            n = T * (min(Hg, (a + 1) * wh) - a * wh) * (min(Wg, (b + 1) * ww) - b * ww)
            out.append((off, n))
            off += -(-n // 128) * 128
    return out, off


def _expected_lists(T, Hg, Wg, wh, ww, routes, npool, kvb, nq_pad):
    wins, _ = _window_rows(T, Hg, Wg, wh, ww)
    lists = []
    for w, (off, n) in enumerate(wins):
        blocks = list(range(off // kvb, (off + n) // kvb))
        for j in sorted(routes[w]):
            o2, n2 = wins[j]
            blocks += range(o2 // kvb, (o2 + n2) // kvb)
        blocks += range(nq_pad // kvb, nq_pad // kvb + -(-npool // kvb))
        for _ in range(-(-n // 128)):
            lists.append(blocks)
    return lists


def _run_basa(env, qb, kb, vb, geo):
    bsa, g, torch = env
    T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kvb = (geo[x] for x in
                                                    ("T", "Hg", "Wg", "wh", "ww", "dy", "dx", "ph",
                                                     "pw", "topk", "kvb"))
    q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    plan = bsa.bsa_basa_plan(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kv_block=kvb,
                             want_routes=True)
    outp, _ = bsa.bsa_attn_fwd(plan["qp"], plan["kp"], plan["vp"], plan["idx"], None,
                               plan["count"], 128, kvb)
    out = bsa.bsa_window_unpermute(outp, T, Hg, Wg, wh, ww, dy, dx)
    torch.cuda.synchronize()
    return plan, out


SMALL = [
    dict(T=2, Hg=12, Wg=20, wh=4, ww=6, dy=1, dx=3, ph=5, pw=4, topk=2, kvb=4, d=64, H=2),
    dict(T=2, Hg=12, Wg=20, wh=4, ww=6, dy=-5, dx=17, ph=5, pw=4, topk=2, kvb=8, d=128, H=2),
    dict(T=3, Hg=10, Wg=16, wh=5, ww=8, dy=2, dx=0, ph=2, pw=3, topk=0, kvb=4, d=128, H=1),
    dict(T=1, Hg=16, Wg=16, wh=4, ww=4, dy=3, dx=1, ph=4, pw=4, topk=5, kvb=16, d=64, H=2),
]


@pytest.mark.parametrize("geo", SMALL, ids=lambda x: f"{x['Hg']}x{x['Wg']}w{x['wh']}x{x['ww']}"
                         f"k{x['topk']}d{x['d']}kv{x['kvb']}")
def test_basa_small_matches_oracle(env, geo):
    _check_small(env, geo)


def test_basa_fuzz_geometries(env):
    """Random grids, window sizes (ragged last windows), rolls, pool cells
    and top-k; KV block the largest power of two (up to 16) dividing every
    window's token count and 128."""
    bsa, g, torch = env
    rng = np.random.default_rng(55)
    for case in range(8):
        T = int(rng.integers(1, 4))
        Hg, Wg = int(rng.integers(3, 17)), int(rng.integers(3, 25))
        wh, ww = int(rng.integers(1, Hg + 1)), int(rng.integers(1, Wg + 1))
        wins, _ = _window_rows(T, Hg, Wg, wh, ww)
        kvb = 16
        while any(n % kvb for _, n in wins):
            kvb //= 2
        nwin = len(wins)
        geo = dict(T=T, Hg=Hg, Wg=Wg, wh=wh, ww=ww, dy=int(rng.integers(-Hg, 2 * Hg)),
                   dx=int(rng.integers(-Wg, 2 * Wg)), ph=int(rng.integers(1, Hg + 1)),
                   pw=int(rng.integers(1, Wg + 1)), topk=min(64, int(rng.integers(0, nwin))), kvb=kvb,
                   d=int(rng.choice([64, 128])), H=2)
        _check_small(env, geo)


def _check_small(env, geo):
    bsa, g, torch = env
    g.say(f"case basa small {geo}")
    T, Hg, Wg, wh, ww, dy, dx = (geo[x] for x in ("T", "Hg", "Wg", "wh", "ww", "dy", "dx"))
    ph, pw, topk, kvb, d, H = (geo[x] for x in ("ph", "pw", "topk", "kvb", "d", "H"))
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=Hg * 7 + d + topk)
    plan, out = _run_basa(env, qb, kb, vb, geo)
    N = T * Hg * Wg
    members = obasa.window_members(T, Hg, Wg, wh, ww, dy % Hg, dx % Wg)
    wins, nq_pad = _window_rows(T, Hg, Wg, wh, ww)
    assert plan["Nq_pad"] == nq_pad and plan["nwin"] == len(members)
    qp = plan["qp"].view(torch.int16).cpu().numpy().view(np.uint16)
    kp = plan["kp"].view(torch.int16).cpu().numpy().view(np.uint16)
    vp = plan["vp"].view(torch.int16).cpu().numpy().view(np.uint16)
    idx = plan["idx"].cpu().numpy()
    cnt = plan["count"].cpu().numpy()
    routes = plan["routes"].cpu().numpy() if topk else None
    got = g.from_dev_bf16(out)
    for h in range(H):
        q32, k32 = bf16_bits_to_f32(qb[0, h]), bf16_bits_to_f32(kb[0, h])
        want_routes = obasa.route(q32, k32, members, topk) if topk else np.zeros((len(members), 0), int)
        if topk:
            np.testing.assert_array_equal(routes[0, h], want_routes)
        # window-major copies and zero pad rows
        for w, (off, n) in enumerate(wins):
            pad = -(-n // 128) * 128
            for src, dst in ((qb, qp), (kb, kp), (vb, vp)):
                np.testing.assert_array_equal(dst[0, h, off:off + n], src[0, h, members[w]])
                assert not dst[0, h, off + n:off + pad].any()
        # pooled memory within one bf16 step (8 significant bits) of the fp64 cell means
        npool = T * -(-Hg // ph) * -(-Wg // pw)
        for src, dst in ((kb, kp), (vb, vp)):
            gm = obasa.pooled_memory(bf16_bits_to_f64(src[0, h]), T, Hg, Wg, ph, pw)
            dev = bf16_bits_to_f64(dst[0, h, nq_pad:])
            assert dev.shape == gm.shape == (npool, d)
            ulp = np.ldexp(1.0, np.frexp(gm)[1] - 8)
            assert (np.abs(dev - gm) <= ulp).all()
        # block lists
        lists = _expected_lists(T, Hg, Wg, wh, ww, want_routes, npool, kvb, nq_pad)
        assert len(lists) == idx.shape[2]
        for i, blocks in enumerate(lists):
            assert cnt[0, h, i] == len(blocks)
            np.testing.assert_array_equal(idx[0, h, i, :len(blocks)], blocks)
            assert (idx[0, h, i, len(blocks):] == -1).all()
        want, _ = obasa.basa_attn(qb[0, h], kb[0, h], vb[0, h], T, Hg, Wg, wh, ww, dy % Hg,
                                  dx % Wg, ph, pw, topk, routes=want_routes)
        assert not np.isnan(want).any()
        g.assert_attn_close(got[0, h], want, f"basa small head {h}")
    assert got.shape == (1, H, N, d)


FULL = {
    # name: (windows sampled, windows, padded query rows)
    "basa_1664x960": ([0, 10, 37, 65], 66, 135936),
    "basa_1664x960_p2": ([0, 37, 65], 66, 135936),
    "basa_1664x960_w15x26": ([0, 15], 16, 131072),
}


@pytest.mark.parametrize("name", list(FULL))
def test_basa_full_size_sampled_windows(env, name):
    """The 1664x960 / 81-frame latent (21 x 60 x 104), one head, Delta =
    (3, 7), top-2 routing: w = (10, 10) with 4 x 4 or 2 x 2 pooling, and
    w = (15, 26) with 4 x 4 pooling (KV block 2).  Routes of every window
    exact, output rows of sampled windows (full, ragged last column, last)
    against the oracle."""
    bsa, g, torch = env
    c = CONFIGS[name]
    wins, nwin, nq_pad = FULL[name]
    geo = dict(T=c["T"], Hg=c["Hg"], Wg=c["Wg"], wh=c["wh"], ww=c["ww"], dy=c["dy"], dx=c["dx"],
               ph=c["ph"], pw=c["pw"], topk=c["topk"], kvb=c["kv_block"])
    g.say(f"case basa full size {name} {geo}")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=11)
    plan, out = _run_basa(env, qb, kb, vb, geo)
    assert plan["nwin"] == nwin and plan["Nq_pad"] == nq_pad
    cnt = plan["count"].cpu().numpy()
    assert cnt.max() <= plan["max_blocks"]
    members = obasa.window_members(c["T"], c["Hg"], c["Wg"], c["wh"], c["ww"], c["dy"], c["dx"])
    want_routes = obasa.route(bf16_bits_to_f32(qb[0, 0]), bf16_bits_to_f32(kb[0, 0]), members,
                              c["topk"])
    np.testing.assert_array_equal(plan["routes"].cpu().numpy()[0, 0], want_routes)
    got = g.from_dev_bf16(out)[0, 0]
    want, _ = obasa.basa_attn(qb[0, 0], kb[0, 0], vb[0, 0], c["T"], c["Hg"], c["Wg"], c["wh"],
                              c["ww"], c["dy"], c["dx"], c["ph"], c["pw"], c["topk"],
                              windows=wins, routes=want_routes)
    rows = np.concatenate([members[w] for w in wins])
    g.assert_attn_close(got[rows], want[rows], f"basa {name} sampled windows")


def _route_job(c, h):
    sh = _pool.shared
    members = obasa.window_members(c["T"], c["Hg"], c["Wg"], c["wh"], c["ww"], c["dy"], c["dx"])
    return obasa.route(bf16_bits_to_f32(sh["qb"][0, h]), bf16_bits_to_f32(sh["kb"][0, h]),
                       members, c["topk"])


def _window_job(c, h, wins):
    """Oracle output rows of windows `wins` of head h against the device's:
    (max-abs, mean-abs) per window."""
    sh = _pool.shared
    want, _ = obasa.basa_attn(sh["qb"][0, h], sh["kb"][0, h], sh["vb"][0, h], c["T"], c["Hg"],
                              c["Wg"], c["wh"], c["ww"], c["dy"], c["dx"], c["ph"], c["pw"],
                              c["topk"], windows=wins, routes=sh["routes"][h])
    members = obasa.window_members(c["T"], c["Hg"], c["Wg"], c["wh"], c["ww"], c["dy"], c["dx"])
    got = bf16_bits_to_f64(sh["out"][0, h])
    out = []
    for w in wins:
        diff = np.abs(got[members[w]] - want[members[w]])
        out.append((h, w, float(diff.max()), float(diff.mean())))
    return out


def test_basa_full_size_two_full_heads():
    """The 1664x960 / 81-frame workload as the benchmark runs it: all 12
    heads of 21 x 60 x 104 tokens in one call per stage, w = (10, 10),
    Delta = (3, 7), top-2 routing, 4 x 4 pooling.  Routes of every window
    of every head exact; output rows of every window of two full heads (the
    first and the last: 2 x 66 windows) against the definition-based
    oracle, within the attention tolerances per window."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu as g
    c = CONFIGS["basa_1664x960"]
    H = c["H"]
    geo = dict(T=c["T"], Hg=c["Hg"], Wg=c["Wg"], wh=c["wh"], ww=c["ww"], dy=c["dy"], dx=c["dx"],
               ph=c["ph"], pw=c["pw"], topk=c["topk"], kvb=c["kv_block"])
    g.say(f"case basa full size, {H} heads, two full heads checked: {geo}")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], H, c["d"], seed=0, workers=_pool.workers())
    plan, out = _run_basa((bsa, g, torch), qb, kb, vb, geo)
    sh = _pool.shared
    sh.clear()
    sh.update(qb=qb, kb=kb, vb=vb, out=out.view(torch.int16).cpu().numpy().view(np.uint16))
    routes = plan["routes"].cpu().numpy()
    del plan, out
    try:
        want = _pool.run(_route_job, [(c, h) for h in range(H)], "basa routes")
        for h in range(H):
            np.testing.assert_array_equal(routes[0, h], want[h])
        sh["routes"] = want
        jobs = [(c, h, list(range(w, min(66, w + 6)))) for h in (0, H - 1) for w in range(0, 66, 6)]
        res = [x for r in _pool.run(_window_job, jobs, "basa windows") for x in r]
    finally:
        sh.clear()
    assert len(res) == 2 * 66
    mx, mean = max(x[2] for x in res), max(x[3] for x in res)
    g.say(f"  basa 2 x 66 windows: max-abs {mx:.3e}, worst window mean-abs {mean:.3e}")
    assert mx <= g.ATTN_MAX_ABS and mean <= g.ATTN_MEAN_ABS


def test_basa_layer_schedule(env):
    """Per-layer structured plans: four layers (each with its own
    activations) at two denoising steps with step offsets, the roll of each
    (layer, step) from bsa_basa_shifts (checked equal to the oracle's
    schedule); each layer's plan, attention and un-permute against the
    oracle at the oracle's own roll."""
    bsa, g, torch = env
    T, Hg, Wg, wh, ww, ph, pw, topk, kvb, d, L, S = 2, 12, 20, 4, 6, 5, 4, 2, 4, 64, 4, 2
    ch, cw = [0, 1], [0, -2]
    dy, dx = bsa.bsa_basa_shifts(wh, ww, L, S, ch, cw)
    bh, bw = obasa.shift_offsets(wh, L), obasa.shift_offsets(ww, L)
    for l in range(L):
        for s in range(S):
            oy, ox = obasa.layer_step_shift(bh, bw, ch, cw, l, s, wh, ww)
            assert (dy[l][s], dx[l][s]) == (oy, ox)
            g.say(f"case basa layer {l} step {s}: Delta = ({oy}, {ox})")
            qb, kb, vb = make_qkv(T, Hg, Wg, 1, d, seed=100 + l)
            geo = dict(T=T, Hg=Hg, Wg=Wg, wh=wh, ww=ww, dy=dy[l][s], dx=dx[l][s], ph=ph, pw=pw,
                       topk=topk, kvb=kvb)
            plan, out = _run_basa(env, qb, kb, vb, geo)
            members = obasa.window_members(T, Hg, Wg, wh, ww, oy, ox)
            routes = obasa.route(bf16_bits_to_f32(qb[0, 0]), bf16_bits_to_f32(kb[0, 0]), members,
                                 topk)
            np.testing.assert_array_equal(plan["routes"].cpu().numpy()[0, 0], routes)
            want, _ = obasa.basa_attn(qb[0, 0], kb[0, 0], vb[0, 0], T, Hg, Wg, wh, ww, oy, ox,
                                      ph, pw, topk, routes=routes)
            g.assert_attn_close(g.from_dev_bf16(out)[0, 0], want, f"layer {l} step {s}")


def test_basa_routing_ties_on_the_device(env):
    """Constructed windows whose relevance ties exactly (the pin of the
    oracle's tie rule): the device routes equal the stated order -- best
    first, equal scores by the lowest window id."""
    bsa, g, torch = env
    from tests.test_oracle_basa import _tie_inputs
    from synth import f64_to_bf16_bits
    g.say("case basa routing ties")
    q, k, mem = _tie_inputs(d=64)
    qb = f64_to_bf16_bits(q.astype(np.float64))[None, None]
    kb = f64_to_bf16_bits(k.astype(np.float64))[None, None]
    for topk, expect in ((3, [1, 2, 4]), (6, [1, 2, 4, 7, 5, 8])):
        geo = dict(T=1, Hg=12, Wg=12, wh=4, ww=4, dy=0, dx=0, ph=4, pw=4, topk=topk, kvb=4)
        plan, _ = _run_basa(env, qb, kb, kb, geo)
        routes = plan["routes"].cpu().numpy()[0, 0]
        want = obasa.route(q, k, mem, topk)
        np.testing.assert_array_equal(routes, want)
        assert routes[0].tolist() == expect
