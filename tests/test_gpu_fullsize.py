"""Full-size parity of the selector -> plan -> attention chain at the pages'
workloads, in the launch configuration the benchmark times (every head of a
workload in one call per stage), against the oracle.

Workloads: the tiny 2 x 32 x 32 case (one cluster, top-8 of 64-token
blocks), Wan2.1-1.3B 480p (SIP 887 of 8,190), Wan2.1-14B 720p (SIP 2048 of
18,900, the benchmark's) and HunyuanVideo 720p (SIP and top-k, 2272 of
29,700); AB-Attention page, sections "어떻게 쓰나" and "전제와 한계".

* P1 scores: every head, every element within 1e-4 relative of the
  oracle's fp64 scores (|S| >= 1e-30); centroids and shares bit-exact
  (both sides take the k-means decisions in the same fp32 order).
* P2 plan, on every row of every head, two ways:
  - the device planner on the oracle's own scores (fp32, as the boundary
    takes them) against the oracle's plan of the same scores;
  - the oracle planner on the device's own scores, widened exactly to fp64,
    against the device's plan of them (the benchmark's chain).
  Indices and counts bit-exact, lambda bitwise, shifts within 2 fp32 ulp.
* P3 attention: the device's attention on its plan of the oracle's scores
  (equal to the oracle's plan by P2) against the oracle's attention on the
  oracle's plan: every query block of every head (ragged last blocks
  included); max-abs <= 2e-2 and mean-abs <= 2e-3 per query block.

The oracle side runs in a pool of forked single-threaded workers (one head
or one run of query blocks per job)."""
import numpy as np
import pytest

from oracle import attn as oat
from oracle import plan as opl
from oracle import select as osel
from synth import CONFIGS, bf16_bits_to_f64, make_qkv
from tests import _pool

pytestmark = pytest.mark.gpu

WORKLOADS = {
    # name: plan modes checked
    "tiny_2x32x32": (opl.TOPK,),
    "wan13b_480p": (opl.SIP,),
    "wan14b_720p": (opl.SIP,),
    "hunyuan_720p": (opl.SIP, opl.TOPK),
}
MODE_NAME = {opl.SIP: "sip", opl.TOPK: "topk"}
SEED = 0


def _cfg(name):
    c = CONFIGS[name]
    N = c["T"] * c["Hg"] * c["Wg"]
    return c, N, -(-N // 128), -(-N // c["kv_block"])


# --------------------------------------------------------------- oracle jobs
def _head_job(name, h):
    """P1 and both P2 checks of head h; returns the oracle's fp32 scores and
    its plans of them (the expected values of the device planner run on
    those scores, and the plans of the oracle's attention)."""
    sh = _pool.shared
    c, N, nqb, M = _cfg(name)
    So, mu, w = osel.select_scores_head(sh["qb"][0, h], sh["kb"][0, h], 128, c["kv_block"],
                                        c["n_clusters"], c["kmeans_iters"])
    Sd = sh["S"][0, h].astype(np.float64)
    keep = np.abs(So) >= 1e-30
    rel = float((np.abs(Sd - So)[keep] / np.abs(So)[keep]).max())
    res = dict(h=h, rel=rel, mu_eq=bool(np.array_equal(sh["mu"][0, h], mu)),
               w_eq=bool(np.array_equal(sh["w"][0, h], w)), So32=So.astype(np.float32))
    for mode in WORKLOADS[name]:
        want = opl.plan(Sd, c["budget"], mode, seed=SEED, row_base=h * nqb)
        res[f"chain_{mode}"] = _plan_diff(sh[f"plan_c{mode}"], h, want)
        res[f"plan_o{mode}"] = opl.plan(So, c["budget"], mode, seed=SEED, row_base=h * nqb)
    return res


def _plan_diff(dev, h, want):
    """(rows whose indices or count differ, rows whose lambda differs
    bitwise, largest shift difference in fp32 ulp) of head h."""
    gi, gb, gc, gl = (x[0, h] for x in dev)
    wi, wb, wc, wl = want
    rows = int(((gi != wi).any(axis=-1) | (gc != wc)).sum())
    lam = int((gl.view(np.int64) != wl.view(np.int64)).sum())
    ulp = np.abs(gb.view(np.int32).astype(np.int64) - wb.view(np.int32).astype(np.int64))
    ulp[np.abs(gb) + np.abs(wb) == 0] = 0
    return rows, lam, int(ulp.max())


def _attn_job(name, mode, h, blocks):
    """Oracle attention of head h on the oracle's plan, for the listed query
    blocks, against the device output: per-block (max-abs, mean-abs)."""
    sh = _pool.shared
    c, N, nqb, M = _cfg(name)
    pi, pb, pc = (x[h] for x in sh[f"plan_o{mode}"])
    q, k, v = (bf16_bits_to_f64(x[0, h]) for x in (sh["qb"], sh["kb"], sh["vb"]))
    ref, _ = oat.attn_fwd(q, k, v, 128, c["kv_block"], pi, None if mode == opl.TOPK else pb, pc,
                          blocks=blocks)
    got = bf16_bits_to_f64(sh[f"out{mode}"][0, h])
    out = []
    for i in blocks:
        r = slice(i * 128, min(N, i * 128 + 128))
        diff = np.abs(got[r] - ref[r])
        out.append((int(i), float(diff.max()), float(diff.mean())))
    return h, out


# --------------------------------------------------------------- device side
_CACHE = {}


def _bits(t, torch):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _results(name):
    """Runs the whole check of a workload once (device chain, oracle jobs)
    and keeps only the latest workload's results."""
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()
    _pool.shared.clear()
    import torch
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu as g
    c, N, nqb, M = _cfg(name)
    H, s, kvb, modes = c["H"], c["budget"], c["kv_block"], WORKLOADS[name]
    g.say(f"case full size {name}: drawing inputs (H={H}, N={N})")
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], H, c["d"], seed=SEED,
                          workers=_pool.workers())
    q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
    g.say(f"case full size {name}: device selector and plan on all heads")
    S, mu, w = bsa.bsa_select_scores(q, k, 128, kvb, c["n_clusters"], c["kmeans_iters"],
                                     want_centroids=True)
    sh = _pool.shared
    sh.update(qb=qb, kb=kb, vb=vb, S=S.cpu().numpy(), mu=mu.cpu().numpy(), w=w.cpu().numpy())
    for mode in modes:
        idx, bias, cnt, lam = bsa.bsa_sip_plan(S, s, mode, seed=SEED, want_lambda=True)
        sh[f"plan_c{mode}"] = tuple(x.cpu().numpy() for x in (idx, bias, cnt, lam))
        del idx, bias, cnt, lam
    del S, mu, w
    g.say(f"case full size {name}: oracle selector and plans of every head")
    heads = _pool.run(_head_job, [(name, h) for h in range(H)], f"{name} heads")
    res = dict(heads=heads, modes=modes, H=H, nqb=nqb)
    So = torch.from_numpy(np.stack([r["So32"] for r in heads])[None]).cuda()
    g.say(f"case full size {name}: device plan and attention on the oracle's scores")
    for mode in modes:
        want = [np.stack([r[f"plan_o{mode}"][j] for r in heads])[None] for j in range(4)]
        idx, bias, cnt, lam = bsa.bsa_sip_plan(So, s, mode, seed=SEED, want_lambda=True)
        dev = tuple(x.cpu().numpy() for x in (idx, bias, cnt, lam))
        res[f"pure_{mode}"] = [_plan_diff(dev, h, [x[0, h] for x in want]) for h in range(H)]
        out, _ = bsa.bsa_attn_fwd(q, k, v, idx, None if mode == opl.TOPK else bias, cnt, 128, kvb)
        sh[f"out{mode}"] = _bits(out, torch)
        sh[f"plan_o{mode}"] = tuple(x[0] for x in want[:3])
        del idx, bias, cnt, lam, out
    del So, q, k, v
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    for r in heads:
        del r["So32"]
        for mode in modes:
            del r[f"plan_o{mode}"]
    jobs = [(name, mode, h, list(range(j, min(nqb, j + 64))))
            for mode in modes for h in range(H) for j in range(0, nqb, 64)]
    g.say(f"case full size {name}: oracle attention on {sum(len(j[3]) for j in jobs)} "
          f"query blocks")
    att = _pool.run(_attn_job, jobs, f"{name} attention")
    for (_, mode, _, _), (h, out) in zip(jobs, att):
        res.setdefault(f"attn_{mode}", []).extend((h,) + o for o in out)
    _pool.shared.clear()
    _CACHE[name] = res
    return res


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import _gpu
    yield _gpu
    _CACHE.clear()
    _pool.shared.clear()


@pytest.fixture(scope="module", params=list(WORKLOADS))
def res(request, env):
    """One workload's results; a module-scoped parameter, so pytest runs
    all checks of one workload before the next one is computed."""
    yield request.param, _results(request.param)
    _CACHE.clear()


def test_fullsize_scores_every_head(env, res):
    g = env
    name, res = res
    worst = max(r["rel"] for r in res["heads"])
    g.say(f"  {name}: {res['H']} heads, scores max rel {worst:.3e}")
    assert worst <= g.SCORE_REL
    assert all(r["mu_eq"] and r["w_eq"] for r in res["heads"]), "centroids or shares differ"


def test_fullsize_plan_every_row_on_oracle_scores(env, res):
    g = env
    name, res = res
    for mode in res["modes"]:
        d = res[f"pure_{mode}"]
        g.say(f"  {name} {MODE_NAME[mode]}: {res['H'] * res['nqb']} rows, rows differing "
              f"{sum(x[0] for x in d)}, lambda differing {sum(x[1] for x in d)}, "
              f"shift ulp {max(x[2] for x in d)}")
        assert sum(x[0] for x in d) == 0 and sum(x[1] for x in d) == 0
        assert max(x[2] for x in d) <= 2


def test_fullsize_plan_every_row_on_device_scores(env, res):
    g = env
    name, res = res
    for mode in res["modes"]:
        d = [r[f"chain_{mode}"] for r in res["heads"]]
        g.say(f"  {name} {MODE_NAME[mode]} (device scores): rows differing "
              f"{sum(x[0] for x in d)}, lambda differing {sum(x[1] for x in d)}, "
              f"shift ulp {max(x[2] for x in d)}")
        assert sum(x[0] for x in d) == 0 and sum(x[1] for x in d) == 0
        assert max(x[2] for x in d) <= 2


def test_fullsize_attention_every_block(env, res):
    g = env
    name, res = res
    for mode in res["modes"]:
        a = res[f"attn_{mode}"]
        mx = max(x[2] for x in a)
        mean = max(x[3] for x in a)
        heads = sorted({x[0] for x in a})
        g.say(f"  {name} {MODE_NAME[mode]}: {len(a)} query blocks over {len(heads)} heads, "
              f"max-abs {mx:.3e}, worst block mean-abs {mean:.3e}")
        assert len(heads) == res["H"] and len(a) == res["H"] * res["nqb"]
        assert mx <= g.ATTN_MAX_ABS and mean <= g.ATTN_MEAN_ABS
