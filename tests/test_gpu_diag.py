"""GPU parity of the accuracy diagnostics (bsa_block_mass, bsa_plan_coverage,
bsa_output_error) against oracle/diag.py.

Block masses: within 1e-4 relative (+1e-30 absolute) of the oracle's fp64
masses, which use their own fp64 normaliser (the device gets the
normaliser rounded to fp32); rows sum to 1 within 1e-4.  Coverage:
bit-exact (fp64 sums in list order on both sides).  Error sums: 1e-12
relative (fp64 sums in different orders)."""
import numpy as np
import pytest

from oracle import diag as odg
from synth import CONFIGS, bf16_bits_to_f64, head_qkv, make_qkv, positional_features

pytestmark = pytest.mark.gpu

MASS_REL = 1e-4
MASS_ABS = 1e-30


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def _check_mass(g, got, want, what):
    ok = ~np.isnan(want)
    err = np.abs(got.astype(np.float64) - want)[ok]
    bound = (MASS_REL * want + MASS_ABS)[ok]
    worst = float((err / bound).max())
    g.say(f"  {what}: max err/bound {worst:.3f}")
    assert worst <= 1.0, f"{what}: error {worst} x the bound"


@pytest.mark.parametrize("B,H,Nq,Nk,d,kvb", [
    (1, 2, 300, 2500, 128, 4),      # ragged query block, ragged last tile
    (1, 1, 200, 9000, 128, 4),      # three key chunks
    (1, 1, 130, 9000, 64, 3),       # three chunks (3582 keys each)
    (1, 2, 128, 1000, 64, 3),       # block size not a power of two
    (2, 1, 200, 777, 128, 128),
    (1, 2, 64, 20, 128, 1),         # fewer keys than one tile
    (1, 1, 130, 3000, 128, 1024),   # one block per chunk
    (1, 2, 129, 1100, 64, 7),
    (1, 1, 1, 5, 128, 4),
])
def test_block_mass_matches_oracle(env, B, H, Nq, Nk, d, kvb):
    bsa, g, torch = env
    g.say(f"case block mass B={B} H={H} Nq={Nq} Nk={Nk} d={d} kv={kvb}")
    qb = np.concatenate([make_qkv(1, 1, Nq, H, d, seed=10 + b)[0] for b in range(B)])
    kb = np.concatenate([make_qkv(1, 1, Nk, H, d, seed=20 + b)[1] for b in range(B)])
    q64, k64 = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb)
    lse = np.stack([[odg.dense_lse(q64[b, h], k64[b, h]) for h in range(H)] for b in range(B)])
    mass = bsa.bsa_block_mass(g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.dev_f32(lse), 128, kvb)
    torch.cuda.synchronize()
    got = mass.cpu().numpy()
    assert got.shape == (B, H, -(-Nq // 128), -(-Nk // kvb))
    for b in range(B):
        for h in range(H):
            want = odg.block_mass(q64[b, h], k64[b, h], 128, kvb)
            _check_mass(g, got[b, h], want, f"b{b} h{h}")
            np.testing.assert_allclose(got[b, h].sum(axis=1, dtype=np.float64), 1.0, rtol=MASS_REL)


def test_block_mass_deterministic(env):
    bsa, g, torch = env
    g.say("case block mass determinism")
    qb, kb, _ = make_qkv(1, 10, 70, 2, 128, seed=3)
    q64, k64 = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb)
    lse = g.dev_f32(np.stack([[odg.dense_lse(q64[0, h], k64[0, h]) for h in range(2)]]))
    q, k = g.to_dev_bf16(qb), g.to_dev_bf16(kb)
    a1 = bsa.bsa_block_mass(q, k, lse, 128, 4).cpu().numpy()
    a2 = bsa.bsa_block_mass(q, k, lse, 128, 4).cpu().numpy()
    assert np.array_equal(a1.view(np.uint32), a2.view(np.uint32))


@pytest.mark.parametrize("kvb", [4, 128])
def test_block_mass_full_size(env, kvb):
    """Wan2.1-14B 720p latent (21 x 45 x 80), head 0: the normaliser comes
    from a dense bsa_attn_fwd call; every row sums to 1 and sampled query
    blocks (first, second, middle, ragged last) match the oracle."""
    bsa, g, torch = env
    c = CONFIGS["wan14b_720p"]
    g.say(f"case block mass full size kv={kvb}")
    phi = positional_features(c["T"], c["Hg"], c["Wg"])
    qh, kh, vh = head_qkv(c["T"], c["Hg"], c["Wg"], c["d"], 0, 0, phi)
    q, k, v = (g.to_dev_bf16(x[None, None]) for x in (qh, kh, vh))
    N = q.shape[2]
    idx, cnt = bsa.dense_plan(1, 1, N, N, 128)
    _, lse = bsa.bsa_attn_fwd(q, k, v, idx, None, cnt, 128, 128, want_lse=True)
    mass = bsa.bsa_block_mass(q, k, lse, 128, kvb)
    torch.cuda.synchronize()
    got = mass.cpu().numpy()[0, 0]
    np.testing.assert_allclose(got.sum(axis=1, dtype=np.float64), 1.0, rtol=MASS_REL)
    rows = [0, 1, 295, got.shape[0] - 1]
    want = odg.block_mass(bf16_bits_to_f64(qh), bf16_bits_to_f64(kh), 128, kvb, blocks=rows)
    _check_mass(g, got[rows], want[rows], f"full size kv={kvb} blocks {rows}")


def test_plan_coverage_bit_exact(env):
    bsa, g, torch = env
    g.say("case plan coverage")
    rng = np.random.default_rng(4)
    rows, M, L = 300, 777, 50
    mass = rng.gamma(0.3, size=(rows, M)).astype(np.float32)
    idx = rng.integers(-3, M + 3, size=(rows, L)).astype(np.int32)
    cnt = rng.integers(-2, L + 5, size=rows).astype(np.int32)
    cov = bsa.bsa_plan_coverage(g.dev_f32(mass), g.dev_i32(idx), g.dev_i32(cnt))
    torch.cuda.synchronize()
    want = odg.plan_coverage(mass, idx, cnt)
    assert np.array_equal(cov.cpu().numpy(), want)


def test_output_error_sums(env):
    bsa, g, torch = env
    g.say("case output error sums")
    B, H, N, d = 2, 3, 1000, 128
    a, _, _ = make_qkv(1, 1, N, B * H, d, seed=5)
    b, _, _ = make_qkv(1, 1, N, B * H, d, seed=6)
    a, b = a.reshape(B, H, N, d), b.reshape(B, H, N, d)
    sums = bsa.bsa_output_error(g.to_dev_bf16(a), g.to_dev_bf16(b))
    torch.cuda.synchronize()
    got = sums.cpu().numpy()
    for i in range(B):
        for h in range(H):
            num, den = odg.output_error(bf16_bits_to_f64(a[i, h]), bf16_bits_to_f64(b[i, h]))
            np.testing.assert_allclose(got[i, h], [num, den], rtol=1e-12)
    same = bsa.bsa_output_error(g.to_dev_bf16(a), g.to_dev_bf16(a)).cpu().numpy()
    assert (same[..., 0] == 0).all()


def test_accuracy_driver_matches_oracle(env):
    """The diagnostics driver on a 2 x 16 x 24 grid (768 tokens, two heads,
    256-token budget) against the same quantities computed by the oracle:
    dense reference, oracle top-k retained mass at three block sizes, and
    the output error of SIP (with and without its weighting), uniform
    sampling and the oracle top-k at 4-token blocks."""
    bsa, g, torch = env
    from block_sparse_attention_mean_amd import accuracy as acc
    from oracle import attn as oat
    from oracle import plan as opl
    from oracle import select as osel
    g.say("case accuracy driver")
    T, Hg, Wg, H, d, tokens, seed = 2, 16, 24, 2, 128, 256, 3
    N = T * Hg * Wg
    nqb, M4 = -(-N // 128), N // 4
    s4 = tokens // 4
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=12)
    q, k, v = (g.to_dev_bf16(x) for x in (qb, kb, vb))
    ref, lse = acc.dense_reference(q, k, v)
    curve = acc.oracle_topk_curve(q, k, lse, tokens, kv_blocks=(64, 16, 4))
    var = acc.variants(q, k, v, ref, lse, tokens, seed=seed, kv_sweep=(32, 4))
    torch.cuda.synchronize()
    w = np.full(nqb, 128.0) / N
    w[-1] = (N - 128 * (nqb - 1)) / N
    refh = g.from_dev_bf16(ref)

    def close(got, want, what):
        g.say(f"  {what}: device {got:.5f} oracle {want:.5f}")
        assert abs(got - want) <= 0.01 + 0.02 * want, what

    for h in range(H):
        q64, k64, v64 = (bf16_bits_to_f64(x[0, h]) for x in (qb, kb, vb))
        dense, _ = oat.dense_attn(q64, k64, v64)
        g.assert_attn_close(refh[0, h], dense, f"head {h} dense reference")
        for b in (64, 16, 4):
            A = odg.block_mass(q64, k64, 128, b)
            oi, oc = odg.oracle_topk(A, max(1, min(A.shape[1], round(tokens / b))))
            cov = float((odg.plan_coverage(A, oi, oc) * w).sum())
            assert abs(curve[b][0, h] - cov) <= 1e-4 * cov, (h, b, curve[b][0, h], cov)
        A4 = odg.block_mass(q64, k64, 128, 4)
        S, _, _ = osel.select_scores_head(qb[0, h], kb[0, h], 128, 4, 8, 1)
        idx, bias, cnt, _ = opl.plan(S, s4, opl.SIP, seed=seed, row_base=h * nqb)
        oi4, oc4 = odg.oracle_topk(A4, s4)
        plans = {
            "ibcs_sip": (idx, bias, cnt),
            "ibcs_sip_no_weighting": (idx, None, cnt),
            "uniform_sampling": opl.plan(np.ones((nqb, M4)), s4, opl.SIP, seed=seed,
                                         row_base=h * nqb)[:3],
            "oracle_topk": (oi4, None, oc4),
        }
        for name, (pi, pb, pc) in plans.items():
            O, _ = oat.attn_fwd(q64, k64, v64, 128, 4, pi, pb, pc)
            close(var[name]["error"][0, h], odg.relative_error(O, dense), f"head {h} {name} error")
            cov = float((odg.plan_coverage(A4, pi, pc) * w).sum())
            close(var[name]["retained_mass"][0, h], cov, f"head {h} {name} retained mass")
