"""Batch dimension B > 1 through every entry point: selector, SIP plan (its
per-row sampling offsets depend on the row's global number (b H + h) nQB + i),
attention and the BASA lists, each (b, h) checked against the oracle."""
import numpy as np
import pytest

from oracle import attn as oat
from oracle import basa as obasa
from oracle import plan as opl
from oracle import select as osel
from synth import bf16_bits_to_f32, bf16_bits_to_f64, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


@pytest.mark.parametrize("d,kvb,Wg", [(128, 4, 37), (128, 2, 37), (64, 4, 38)])
def test_batch_select_plan_attention(env, d, kvb, Wg):
    """Scores of every (b, h) against the oracle's; then the oracle's scores
    go through the device plan and attention (the oracle sees only its own
    values), which must match the oracle's plan and attention.  KV blocks of
    2 tokens at d = 128 and 4 at d = 64 run the half-load gather."""
    bsa, g, torch = env
    B, H, T, Hg, C, budget = 2, 3, 2, 9, 8, 40
    g.say(f"case batch path B={B} H={H} N={T * Hg * Wg} d={d} kv_block={kvb}")
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=21, B=B)
    q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    S, _, _ = bsa.bsa_select_scores(q, k, 128, kvb, C, 1)
    torch.cuda.synchronize()
    Sg = S.cpu().numpy()
    nqb = Sg.shape[2]
    So = np.empty(Sg.shape, np.float64)
    for b in range(B):
        for h in range(H):
            So[b, h], _, _ = osel.select_scores_head(qb[b, h], kb[b, h], 128, kvb, C, 1)
            rel = np.abs(Sg[b, h] - So[b, h]) / np.maximum(np.abs(So[b, h]), 1e-30)
            assert rel[np.abs(So[b, h]) >= 1e-30].max() <= g.SCORE_REL, (b, h)
    idx, bias, cnt, lam = bsa.bsa_sip_plan(g.dev_f32(So), budget, bsa.PLAN_SIP, seed=5,
                                           want_lambda=True)
    out, _ = bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb)
    torch.cuda.synchronize()
    got_out = g.from_dev_bf16(out)
    for b in range(B):
        for h in range(H):
            wi, wb, wc, wl = opl.plan(So[b, h], budget, opl.SIP, seed=5,
                                      row_base=(b * H + h) * nqb)
            np.testing.assert_array_equal(cnt[b, h].cpu().numpy(), wc)
            np.testing.assert_array_equal(idx[b, h].cpu().numpy(), wi)
            np.testing.assert_array_equal(lam[b, h].cpu().numpy(), wl)
            ref, _ = oat.attn_fwd(*(bf16_bits_to_f64(x[b, h]) for x in (qb, kb, vb)), 128, kvb,
                                  wi, wb, wc)
            g.assert_attn_close(got_out[b, h], ref, f"batch b={b} h={h}")


def test_batch_basa(env):
    bsa, g, torch = env
    B, H, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kvb, d = 2, 2, 2, 12, 20, 4, 6, 1, 3, 5, 4, 2, 4, 64
    g.say(f"case batch basa B={B} H={H}")
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=33, B=B)
    q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    plan = bsa.bsa_basa_plan(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kv_block=kvb,
                             want_routes=True)
    outp, _ = bsa.bsa_attn_fwd(plan["qp"], plan["kp"], plan["vp"], plan["idx"], None,
                               plan["count"], 128, kvb)
    out = bsa.bsa_window_unpermute(outp, T, Hg, Wg, wh, ww, dy, dx)
    torch.cuda.synchronize()
    got = g.from_dev_bf16(out)
    routes = plan["routes"].cpu().numpy()
    members = obasa.window_members(T, Hg, Wg, wh, ww, dy, dx)
    for b in range(B):
        for h in range(H):
            want_routes = obasa.route(bf16_bits_to_f32(qb[b, h]), bf16_bits_to_f32(kb[b, h]),
                                      members, topk)
            np.testing.assert_array_equal(routes[b, h], want_routes)
            want, _ = obasa.basa_attn(qb[b, h], kb[b, h], vb[b, h], T, Hg, Wg, wh, ww, dy, dx,
                                      ph, pw, topk, routes=want_routes)
            g.assert_attn_close(got[b, h], want, f"batch basa b={b} h={h}")
