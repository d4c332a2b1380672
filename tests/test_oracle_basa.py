"""Pins of the BASA-structured oracle: the shift-schedule worked example, the
own-window special case against a torch.roll window partition (Swin style),
roll/unroll identity, pooled memory, and routing by brute force."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import basa as ob
from synth import bf16_bits_to_f32, bf16_bits_to_f64, make_qkv


def test_shift_schedule_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "basa_shift_schedule.json")))
    delta = max(1, g["w"] // g["L"])
    assert [(i * delta) % g["w"] for i in range(g["L"])] == g["candidates"]
    assert ob.shift_offsets(g["w"], g["L"]) == g["interleaved"]


@pytest.mark.parametrize("w,L", [(8, 4), (10, 5), (10, 10), (26, 30), (15, 4), (1, 3), (7, 1)])
def test_shift_schedule_properties(w, L):
    """The interleave only reorders the candidates; even positions carry the
    first half in order and odd positions the second half; with L <= w the
    offsets are distinct multiples of delta; with L > w they cycle."""
    delta = max(1, w // L)
    cand = [(i * delta) % w for i in range(L)]
    b = ob.shift_offsets(w, L)
    K = -(-L // 2)
    assert sorted(b) == sorted(cand) and len(b) == L
    assert b[0::2] == cand[:K] and b[1::2] == cand[K:]
    if L <= w:
        assert len(set(b)) == L and all(x % delta == 0 for x in b)
    else:
        assert set(b) == set(range(w))


def test_layer_step_shift():
    bh, bw = ob.shift_offsets(10, 4), ob.shift_offsets(26, 4)
    ch, cw = [0, 3, -4], [5, 0, 30]
    for l in range(4):
        assert ob.layer_step_shift(bh, bw, [0], [0], l, 0, 10, 26) == (bh[l], bw[l])
        for s in range(3):
            dy, dx = ob.layer_step_shift(bh, bw, ch, cw, l, s, 10, 26)
            assert 0 <= dy < 10 and 0 <= dx < 26
            assert (dy - bh[l] - ch[s]) % 10 == 0 and (dx - bw[l] - cw[s]) % 26 == 0


def test_windows_partition_tokens():
    T, Hg, Wg = 3, 12, 14
    mem = ob.window_members(T, Hg, Wg, 5, 4, 3, 7)
    allt = np.concatenate(mem)
    assert np.array_equal(np.sort(allt), np.arange(T * Hg * Wg))
    wid = ob.window_of_token(T, Hg, Wg, 5, 4, 3, 7)
    for w, m in enumerate(mem):
        assert np.all(wid[m] == w)


def test_roll_unroll_identity():
    x = torch.arange(2 * 6 * 10).reshape(2, 6, 10)
    y = torch.roll(torch.roll(x, shifts=(-3, -7), dims=(1, 2)), shifts=(3, 7), dims=(1, 2))
    assert torch.equal(x, y)


def _swin_reference(q, k, v, T, Hg, Wg, wh, ww, dy, dx):
    """Roll by -Delta, cut windows (all frames), SDPA per window, roll back."""
    d = q.shape[1]
    out = torch.zeros(T, Hg, Wg, d, dtype=torch.float64)
    grids = [torch.roll(torch.from_numpy(x).reshape(T, Hg, Wg, d), shifts=(-dy, -dx), dims=(1, 2))
             for x in (q, k, v)]
    for a in range(0, Hg, wh):
        for b in range(0, Wg, ww):
            tq, tk, tv = (g[:, a:a + wh, b:b + ww].reshape(1, 1, -1, d) for g in grids)
            o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
            out[:, a:a + wh, b:b + ww] = o.reshape(T, -1, min(ww, Wg - b), d)
    return torch.roll(out, shifts=(dy, dx), dims=(1, 2)).reshape(-1, d).numpy()


def test_own_window_only_is_shifted_window_attention():
    T, Hg, Wg, d = 3, 12, 14, 32
    qb, kb, vb = (x[0, 0] for x in make_qkv(T, Hg, Wg, 1, d, seed=2))
    q, k, v = (bf16_bits_to_f64(x) for x in (qb, kb, vb))
    mem = ob.window_members(T, Hg, Wg, 5, 4, 3, 7)
    O = np.zeros_like(q)
    for m in mem:
        lg = q[m] @ k[m].T / np.sqrt(d)
        e = np.exp(lg - lg.max(axis=1, keepdims=True))
        O[m] = (e @ v[m]) / e.sum(axis=1, keepdims=True)
    ref = _swin_reference(q, k, v, T, Hg, Wg, 5, 4, 3, 7)
    np.testing.assert_allclose(O, ref, rtol=1e-11, atol=1e-12)


def test_pooled_memory_means():
    rng = np.random.default_rng(0)
    T, Hg, Wg, d = 2, 8, 12, 4
    x = rng.standard_normal((T * Hg * Wg, d))
    assert np.array_equal(ob.pooled_memory(x, T, Hg, Wg, 1, 1), x)
    g = ob.pooled_memory(x, T, Hg, Wg, 4, 4)
    assert g.shape == (T * 2 * 3, d)
    grid = x.reshape(T, Hg, Wg, d)
    np.testing.assert_allclose(g[1 * 6 + 1 * 3 + 2], grid[1, 4:8, 8:12].mean(axis=(0, 1)))


def test_routing_brute_force():
    T, Hg, Wg, d = 2, 20, 20, 16
    qb, kb, _ = (x[0, 0] for x in make_qkv(T, Hg, Wg, 1, d, seed=5))
    q32, k32 = bf16_bits_to_f32(qb), bf16_bits_to_f32(kb)
    mem = ob.window_members(T, Hg, Wg, 5, 5, 1, 2)
    routes = ob.route(q32, k32, mem, 2)
    q64, k64 = q32.astype(np.float64), k32.astype(np.float64)
    qd = np.stack([q64[m].mean(axis=0) for m in mem])
    kd = np.stack([k64[m].mean(axis=0) for m in mem])
    sc = qd @ kd.T
    for i in range(len(mem)):
        cand = sorted((j for j in range(len(mem)) if j != i), key=lambda j: (-sc[i, j], j))
        gap = sc[i, cand[1]] - sc[i, cand[2]]
        if gap > 1e-4 and sc[i, cand[0]] - sc[i, cand[1]] > 1e-4:
            assert set(routes[i]) == set(cand[:2])
        assert i not in routes[i]


def test_basa_key_set_definition_small():
    T, Hg, Wg, d = 2, 8, 12, 16
    qb, kb, vb = (x[0, 0] for x in make_qkv(T, Hg, Wg, 1, d, seed=9))
    O, routes = ob.basa_attn(qb, kb, vb, T, Hg, Wg, 4, 4, 1, 3, 4, 4, 2)
    q, k, v = (bf16_bits_to_f64(x) for x in (qb, kb, vb))
    mem = ob.window_members(T, Hg, Wg, 4, 4, 1, 3)
    gk = ob.pooled_memory(k, T, Hg, Wg, 4, 4)
    gv = ob.pooled_memory(v, T, Hg, Wg, 4, 4)
    wid = ob.window_of_token(T, Hg, Wg, 4, 4, 1, 3)
    for n in (0, 17, 100, T * Hg * Wg - 1):
        w = wid[n]
        keys = np.concatenate([mem[w], mem[routes[w][0]], mem[routes[w][1]]])
        kk, vv = np.concatenate([k[keys], gk]), np.concatenate([v[keys], gv])
        lg = kk @ q[n] / 4.0
        p = np.exp(lg - lg.max()); p /= p.sum()
        np.testing.assert_allclose(O[n], p @ vv, rtol=1e-12, atol=1e-13)


def _tie_inputs(d=8):
    """A 1 x 12 x 12 grid cut into nine 4 x 4 windows (no roll) whose key
    descriptors are a_w e_0 + 0.5 (e_1 + ... + e_{d-1}) with a = (2, 3, 3, 1,
    3, 2, 1, 3, 2), and every query all ones: the score of candidate w is
    a_w + 0.5 (d - 1) for every query window, exactly, in fp32 -- four
    windows tie at the top, three below them, two at the bottom."""
    T, Hg, Wg = 1, 12, 12
    a = np.array([2, 3, 3, 1, 3, 2, 1, 3, 2], np.float32)
    mem = ob.window_members(T, Hg, Wg, 4, 4, 0, 0)
    q = np.ones((T * Hg * Wg, d), np.float32)
    k = np.full((T * Hg * Wg, d), 0.5, np.float32)
    for w, m in enumerate(mem):
        k[m, 0] = a[w]
    return q, k, mem


@pytest.mark.parametrize("topk,expect", [
    (3, {0: [1, 2, 4], 1: [2, 4, 7], 2: [1, 4, 7], 3: [1, 2, 4], 4: [1, 2, 7],
         5: [1, 2, 4], 6: [1, 2, 4], 7: [1, 2, 4], 8: [1, 2, 4]}),
    (6, {0: [1, 2, 4, 7, 5, 8], 1: [2, 4, 7, 0, 5, 8], 5: [1, 2, 4, 7, 0, 8],
         3: [1, 2, 4, 7, 0, 5], 8: [1, 2, 4, 7, 0, 5]}),
])
def test_routing_ties_go_to_the_lowest_window(topk, expect):
    """Equal relevance: rank order best first, and among equal scores the
    lowest window id first (the reading the boundary documents)."""
    q, k, mem = _tie_inputs()
    routes = ob.route(q, k, mem, topk)
    for i, want in expect.items():
        assert routes[i].tolist() == want, (i, routes[i].tolist())
