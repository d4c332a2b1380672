"""Full-size parity at the Wan2.1-14B 720p workload in the launch
configuration the benchmark times: all 40 heads of 75,600 tokens go through
bsa_select_scores -> bsa_sip_plan (SIP, budget 2048, seed 0) ->
bsa_attn_fwd in single calls, then sampled outputs are checked against the
oracle one by one:

* scores: sampled rows of heads 0 and 39 against the oracle's selector;
* plan: sampled rows of three heads, the oracle planning on the GPU's own
  scores (widened exactly) -- indices, counts and lambda bit-exact;
* attention: sampled query blocks of three heads (including the 80-row last
  block) against the oracle on the GPU's plan."""
import os

import numpy as np
import pytest

from oracle import attn as oat
from oracle import plan as opl
from oracle import select as osel
from synth import CONFIGS, bf16_bits_to_f64, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu as g
    c = CONFIGS["wan14b_720p"]
    T, Hg, Wg, H, d, kvb, s = c["T"], c["Hg"], c["Wg"], c["H"], c["d"], c["kv_block"], c["budget"]
    g.say("case full size wan14b_720p: drawing inputs")
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=0, workers=min(16, os.cpu_count() or 1))
    q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    g.say("case full size wan14b_720p: select, plan, attention on all heads")
    S, _, _ = bsa.bsa_select_scores(q, k, 128, kvb, c["n_clusters"], c["kmeans_iters"])
    idx, bias, cnt, lam = bsa.bsa_sip_plan(S, s, bsa.PLAN_SIP, seed=0, want_lambda=True)
    out, _ = bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb)
    torch.cuda.synchronize()
    return dict(c=c, qb=qb, kb=kb, vb=vb, S=S, idx=idx, bias=bias, cnt=cnt, lam=lam, out=out, g=g)


def test_fullsize_scores_sampled_rows(run):
    g, c = run["g"], run["c"]
    for h in (0, 39):
        g.say(f"case full size scores head {h}")
        want, _, _ = osel.select_scores_head(run["qb"][0, h], run["kb"][0, h], 128, c["kv_block"],
                                             c["n_clusters"], c["kmeans_iters"])
        rows = np.r_[0:4, 290:294, 587:591]
        got = run["S"][0, h, rows].cpu().numpy().astype(np.float64)
        ref = want[rows]
        keep = np.abs(ref) >= 1e-30
        rel = np.abs(got - ref)[keep] / np.abs(ref)[keep]
        g.say(f"  max rel {rel.max():.3e}")
        assert rel.max() <= g.SCORE_REL


def test_fullsize_plan_sampled_rows(run):
    g, c = run["g"], run["c"]
    nqb = run["S"].shape[2]
    for h in (0, 17, 39):
        g.say(f"case full size plan head {h}")
        rows = np.r_[0:3, 300:303, nqb - 3:nqb]
        S = run["S"][0, h, rows].cpu().numpy().astype(np.float64)
        # oracle offsets of these rows: the same seeded function, row = h * nQB + i
        offs = np.array([opl.sampling_offset(0, h * nqb + int(i)) for i in rows], dtype=np.uint64)
        want_idx, want_bias, want_cnt, want_lam = opl.plan(S, c["budget"], opl.SIP, offsets=offs)
        got_idx = run["idx"][0, h, rows].cpu().numpy()
        got_cnt = run["cnt"][0, h, rows].cpu().numpy()
        got_bias = run["bias"][0, h, rows].cpu().numpy()
        got_lam = run["lam"][0, h, rows].cpu().numpy()
        np.testing.assert_array_equal(got_cnt, want_cnt)
        np.testing.assert_array_equal(got_idx, want_idx)
        np.testing.assert_array_equal(got_lam, want_lam)
        wb = want_bias.astype(np.float32)
        assert np.all(np.abs(got_bias - wb) <= 2 * np.spacing(np.abs(wb)) + 1e-30)


def test_fullsize_attention_sampled_blocks(run):
    g, c = run["g"], run["c"]
    nqb = run["S"].shape[2]
    rng = np.random.default_rng(7)
    for h in (0, 17, 39):
        blocks = sorted(set(rng.choice(nqb - 1, 7, replace=False).tolist()) | {nqb - 1})
        g.say(f"case full size attention head {h} blocks {blocks}")
        idx = run["idx"][0, h].cpu().numpy()
        bias = run["bias"][0, h].cpu().numpy()
        cnt = run["cnt"][0, h].cpu().numpy()
        q, k, v = (bf16_bits_to_f64(x[0, h]) for x in (run["qb"], run["kb"], run["vb"]))
        ref, _ = oat.attn_fwd(q, k, v, 128, c["kv_block"], idx, bias, cnt, blocks=blocks)
        rows = np.concatenate([np.arange(i * 128, min(q.shape[0], i * 128 + 128)) for i in blocks])
        got = g.from_dev_bf16(run["out"][0, h])
        g.assert_attn_close(got[rows], ref[rows], f"head {h} sampled blocks")
