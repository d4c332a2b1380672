"""GPU parity of bsa_select_scores against the oracle: k-means centroids and
shares bit-exact (both sides take the assignment decisions in the same fp32
order), block scores within 1e-4 relative (|S| >= 1e-30)."""
import numpy as np
import pytest

from oracle import select as osel
from synth import CONFIGS, head_qkv, make_qkv, positional_features

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def _gpu_select(env, qb, kb, kvb, C, iters):
    bsa, g, torch = env
    q, k = g.to_dev_bf16(qb), g.to_dev_bf16(kb)
    S, mu, w = bsa.bsa_select_scores(q, k, 128, kvb, C, iters, want_centroids=True)
    torch.cuda.synchronize()
    return S.cpu().numpy(), mu.cpu().numpy(), w.cpu().numpy()


def _check_head(g, qh, kh, Sg, mug, wg, kvb, C, iters, what):
    S, mu, w = osel.select_scores_head(qh, kh, 128, kvb, C, iters)
    assert np.array_equal(mug.view(np.uint32), mu.view(np.uint32)), f"{what}: centroids differ"
    assert np.array_equal(wg.view(np.uint32), w.view(np.uint32)), f"{what}: shares differ"
    ok = np.abs(S) >= 1e-30
    rel = np.abs(Sg.astype(np.float64) - S)[ok] / np.abs(S[ok])
    g.say(f"  {what}: max rel {rel.max():.3e}")
    assert rel.max() <= g.SCORE_REL, f"{what}: max rel {rel.max()}"


@pytest.mark.parametrize("T,Hg,Wg,d,kvb,C,iters", [
    (1, 8, 16, 64, 4, 8, 1), (1, 10, 100, 128, 4, 8, 1), (2, 8, 40, 128, 16, 4, 2),
    (1, 5, 26, 64, 1, 16, 1), (1, 10, 100, 128, 4, 8, 0), (1, 3, 5, 128, 4, 8, 1),
    (2, 16, 16, 128, 128, 2, 3), (1, 1, 1000, 64, 8, 1, 1),
])
def test_select_matches_oracle_small(env, T, Hg, Wg, d, kvb, C, iters):
    bsa, g, torch = env
    g.say(f"case select T={T} Hg={Hg} Wg={Wg} d={d} kv={kvb} C={C} it={iters}")
    qb, kb, _ = make_qkv(T, Hg, Wg, 2, d, seed=T * Hg + Wg + d)
    Sg, mug, wg = _gpu_select(env, qb, kb, kvb, C, iters)
    for h in range(2):
        _check_head(g, qb[0, h], kb[0, h], Sg[0, h], mug[0, h], wg[0, h], kvb, C, iters, f"head {h}")


def test_select_fuzz_geometries(env):
    """Random sequence lengths (ragged query blocks and ragged 32-block key
    tiles), KV block sizes, cluster counts, head dims and iteration counts,
    two heads each, every output checked."""
    bsa, g, torch = env
    rng = np.random.default_rng(99)
    for case in range(12):
        d = int(rng.choice([64, 128]))
        kvb = int(rng.choice([1, 2, 4, 8, 16, 64]))
        C = int(rng.choice([1, 2, 4, 8, 16]))
        iters = int(rng.integers(0, 3))
        N = int(rng.integers(1, 2500))
        g.say(f"case select fuzz {case}: N={N} d={d} kv={kvb} C={C} it={iters}")
        qb, kb, _ = make_qkv(1, 1, N, 2, d, seed=1000 + case)
        Sg, mug, wg = _gpu_select(env, qb, kb, kvb, C, iters)
        for h in range(2):
            _check_head(g, qb[0, h], kb[0, h], Sg[0, h], mug[0, h], wg[0, h], kvb, C, iters,
                        f"fuzz {case} head {h}")


def test_select_tiny_config_mean_pooled(env):
    bsa, g, torch = env
    c = CONFIGS["tiny_2x32x32"]
    g.say("case select tiny mean-pooled")
    qb, kb, _ = make_qkv(c["T"], c["Hg"], c["Wg"], 1, c["d"], seed=0)
    Sg, mug, wg = _gpu_select(env, qb, kb, c["kv_block"], 1, 1)
    _check_head(g, qb[0, 0], kb[0, 0], Sg[0, 0], mug[0, 0], wg[0, 0], c["kv_block"], 1, 1, "tiny")


@pytest.mark.parametrize("name,heads", [("wan13b_480p", (0, 5, 11)), ("wan14b_720p", (0, 39)),
                                        ("hunyuan_720p", (23,))])
def test_select_full_size_heads(env, name, heads):
    """Full latent shapes; the listed heads of the workload are generated
    with their own per-head seeds and checked completely."""
    bsa, g, torch = env
    c = CONFIGS[name]
    g.say(f"case select full {name} heads {heads}")
    phi = positional_features(c["T"], c["Hg"], c["Wg"])
    hq, hk = [], []
    for h in heads:
        q, k, _ = head_qkv(c["T"], c["Hg"], c["Wg"], c["d"], 0, h, phi)
        hq.append(q)
        hk.append(k)
    qb, kb = np.stack(hq)[None], np.stack(hk)[None]
    Sg, mug, wg = _gpu_select(env, qb, kb, c["kv_block"], c["n_clusters"], c["kmeans_iters"])
    for i, h in enumerate(heads):
        _check_head(g, qb[0, i], kb[0, i], Sg[0, i], mug[0, i], wg[0, i], c["kv_block"],
                    c["n_clusters"], c["kmeans_iters"], f"{name} head {h}")


def test_select_deterministic(env):
    bsa, g, torch = env
    g.say("case select determinism")
    qb, kb, _ = make_qkv(2, 10, 30, 2, 128, seed=1)
    a1 = _gpu_select(env, qb, kb, 4, 8, 1)
    a2 = _gpu_select(env, qb, kb, 4, 8, 1)
    for x, y in zip(a1, a2):
        assert np.array_equal(x, y)
