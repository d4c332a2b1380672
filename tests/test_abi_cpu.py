"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/bsa.h declares, and rejects invalid calls with status codes before
any HIP call (no GPU is touched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_mean_amd as m
    return m


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(bsa):
    declared = _declared_symbols()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(bsa.lib, name), name
    assert sorted(bsa.SYMBOLS) == declared


def test_status_strings(bsa):
    for s in range(-9, 1):
        assert len(bsa.lib.bsa_status_string(s)) > 0
    assert bsa.lib.bsa_status_string(-99) == b"unknown status"
    assert b"gfx950" in bsa.lib.bsa_version()


def test_sampling_offset_matches_oracle(bsa):
    from oracle.splitmix import sampling_offset
    for seed in (0, 1, 12345, 2**64 - 1):
        for row in (0, 1, 2, 99, 23639, 10**9):
            assert bsa.bsa_sampling_offset(seed, row) == sampling_offset(seed, row)


FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced


def _attn(bsa, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, H=1, Nq=256, Nk=256, d=128, qb=128, kvb=4, idx=FAKE,
             bias=None, count=FAKE, L=8, scale=0.0, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return bsa.lib.bsa_attn_fwd(a["q"], a["k"], a["v"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                                a["qb"], a["kvb"], a["idx"], a["bias"], a["count"], a["L"],
                                a["scale"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(idx=None), -1), (dict(out=None), -1), (dict(count=None), -1),
    (dict(B=0), -1), (dict(Nq=0), -1), (dict(Nk=-3), -1), (dict(L=0), -1),
    (dict(scale=float("nan")), -1),
    (dict(d=96), -2), (dict(d=256), -2), (dict(qb=64), -2), (dict(kvb=3), -2), (dict(kvb=256), -2),
    (dict(q=FAKE + 8), -4), (dict(out=FAKE + 2), -4), (dict(idx=FAKE + 2), -4),
    (dict(H=2**20, Nq=2**20 * 4), -7), (dict(L=2**28, kvb=128), -7),
])
def test_attn_fwd_rejects_invalid_arguments(bsa, kw, status):
    assert _attn(bsa, **kw) == status


def _plan(bsa, **kw):
    a = dict(S=FAKE, B=1, H=1, nqb=4, M=100, s=10, mode=0, seed=0, off=None, idx=FAKE, bias=FAKE,
             count=FAKE, lam=None, status=None, stream=None)
    a.update(kw)
    return bsa.lib.bsa_sip_plan(a["S"], a["B"], a["H"], a["nqb"], a["M"], a["s"], a["mode"],
                                a["seed"], a["off"], a["idx"], a["bias"], a["count"], a["lam"],
                                a["status"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=None), -1), (dict(idx=None), -1), (dict(count=None), -1), (dict(M=0), -1),
    (dict(mode=2), -1), (dict(s=0), -3), (dict(s=101), -3), (dict(S=FAKE + 4), -4),
    (dict(lam=FAKE + 4), -4), (dict(status=FAKE + 2), -4), (dict(M=(1 << 20) + 1, s=5), -7),
    (dict(M=(1 << 20) + 1, s=5, mode=1), -7),
    # SIP rows longer than BSA_SIP_MAX_BLOCKS could draw fewer than s blocks
    (dict(M=65025, s=5), -7), (dict(M=2**17, s=2**16), -7),
])
def test_sip_plan_rejects_invalid_arguments(bsa, kw, status):
    assert _plan(bsa, **kw) == status


def test_select_rejects_invalid_arguments(bsa):
    L = bsa.lib
    n = ctypes.c_size_t(0)
    assert L.bsa_select_workspace_bytes(1, 1, 256, 128, 128, 4, 8, None) == -1
    assert L.bsa_select_workspace_bytes(1, 1, 256, 96, 128, 4, 8, ctypes.byref(n)) == -2
    assert L.bsa_select_workspace_bytes(1, 1, 256, 128, 128, 4, 17, ctypes.byref(n)) == -2
    assert L.bsa_select_workspace_bytes(1, 1, 256, 128, 128, 4, 8, ctypes.byref(n)) == 0
    base = (FAKE, FAKE, 1, 1, 256, 128, 128, 4, 8, 1, FAKE, None, None, FAKE, 1 << 30, None)

    def call(i, val):
        a = list(base)
        a[i] = val
        return L.bsa_select_scores(*a)
    assert call(0, None) == -1
    assert call(10, None) == -1
    assert call(9, -1) == -1
    assert call(8, 0) == -2
    assert call(5, 32) == -2
    assert call(0, FAKE + 2) == -4
    assert call(13, None) == -6
    assert call(14, 0) == -6
    assert call(13, FAKE + 16) == -4
    # one head's score matrix must hold fewer than 2^32 entries: N = 750,000
    # at single-token blocks gives 5,860 x 750,000 (refused before any use of
    # the pointers); 100,000 tokens pass the size checks and stop at the
    # one-byte workspace
    big = list(base)
    big[4], big[7], big[14] = 750000, 1, 1
    assert L.bsa_select_scores(*big) == -7
    big[4] = 100000
    assert L.bsa_select_scores(*big) == -6


def test_basa_layout_of_the_1664x960_grid(bsa):
    lay = bsa.bsa_basa_layout(21, 60, 104, 128, 10, 10, 4, 4, 2, 4, 1, 12)
    assert lay["nwin"] == 66
    assert lay["Nq_pad"] == 135936          # 60 windows of 2176 rows + 6 of 896
    assert lay["Nk"] == 135936 + 8190        # + 21 x 15 x 26 pooled tokens
    assert lay["max_blocks"] == 3 * 525 + 2048


def test_basa_rejects_invalid_arguments(bsa):
    with pytest.raises(bsa.BsaError):
        bsa.bsa_basa_layout(21, 60, 104, 96, 10, 10, 4, 4, 2)
    with pytest.raises(bsa.BsaError):
        bsa.bsa_basa_layout(21, 60, 104, 128, 70, 10, 4, 4, 2)
    with pytest.raises(bsa.BsaError):   # 3-token kv blocks are not powers of two
        bsa.bsa_basa_layout(21, 60, 104, 128, 10, 10, 4, 4, 2, kv_block=3)


def _mass(bsa, **kw):
    a = dict(q=FAKE, k=FAKE, lse=FAKE, B=1, H=1, Nq=300, Nk=500, d=128, qb=128, kvb=4, scale=0.0,
             mass=FAKE)
    a.update(kw)
    return bsa.lib.bsa_block_mass(a["q"], a["k"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                                  a["d"], a["qb"], a["kvb"], a["scale"], a["mass"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(mass=None), -1), (dict(Nk=0), -1),
    (dict(kvb=0), -1), (dict(scale=float("inf")), -1),
    (dict(d=96), -2), (dict(qb=64), -2), (dict(kvb=1025), -2),
    (dict(k=FAKE + 8), -4), (dict(lse=FAKE + 2), -4),
    (dict(H=2**16, Nq=2**16, Nk=2**16), -7),
])
def test_block_mass_rejects_invalid_arguments(bsa, kw, status):
    assert _mass(bsa, **kw) == status


def test_coverage_and_error_reject_invalid_arguments(bsa):
    L = bsa.lib
    assert L.bsa_plan_coverage(None, FAKE, FAKE, 4, 10, 3, FAKE, None) == -1
    assert L.bsa_plan_coverage(FAKE, FAKE, FAKE, 0, 10, 3, FAKE, None) == -1
    assert L.bsa_plan_coverage(FAKE, FAKE, FAKE, 4, 10, 3, FAKE + 4, None) == -4
    assert L.bsa_output_error(FAKE, FAKE, 2, 12, FAKE, None) == -1
    assert L.bsa_output_error(FAKE, None, 2, 16, FAKE, None) == -1
    assert L.bsa_output_error(FAKE + 8, FAKE, 2, 16, FAKE, None) == -4


def test_basa_shift_schedule_matches_oracle(bsa):
    from oracle import basa as ob
    assert bsa.bsa_basa_offsets(8, 4) == [0, 4, 2, 6]
    rng = __import__("numpy").random.default_rng(3)
    for w in (1, 2, 7, 8, 10, 15, 26, 32):
        for L in (1, 2, 3, 4, 5, 12, 30, 40):
            assert bsa.bsa_basa_offsets(w, L) == ob.shift_offsets(w, L), (w, L)
    for wh, ww, L, S in ((10, 10, 4, 3), (15, 26, 30, 2), (5, 7, 6, 1)):
        ch = rng.integers(-40, 40, S).tolist()
        cw = rng.integers(-40, 40, S).tolist()
        dy, dx = bsa.bsa_basa_shifts(wh, ww, L, S, ch, cw)
        bh, bw = ob.shift_offsets(wh, L), ob.shift_offsets(ww, L)
        for l in range(L):
            for s in range(S):
                assert (dy[l][s], dx[l][s]) == ob.layer_step_shift(bh, bw, ch, cw, l, s, wh, ww)
        dy0, dx0 = bsa.bsa_basa_shifts(wh, ww, L, S)
        assert all(dy0[l] == [bh[l]] * S and dx0[l] == [bw[l]] * S for l in range(L))


def test_basa_shift_schedule_rejects_invalid_arguments(bsa):
    L = bsa.lib
    buf = (ctypes.c_int * 8)()
    assert L.bsa_basa_offsets(0, 4, buf) == -1
    assert L.bsa_basa_offsets(8, 0, buf) == -1
    assert L.bsa_basa_offsets(8, 4, None) == -1
    assert L.bsa_basa_shifts(10, 10, 2, 0, None, None, buf, buf) == -1
    assert L.bsa_basa_shifts(10, 0, 2, 2, None, None, buf, buf) == -1
    assert L.bsa_basa_shifts(10, 10, 2, 2, None, None, None, buf) == -1


def _bwd(bsa, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, B=1, H=1, Nq=300, Nk=300, d=128,
             qb=128, kvb=4, idx=FAKE, bias=None, cnt=FAKE, L=8, scale=0.0, dq=FAKE,
             dk=FAKE + 4096, dv=FAKE + 8192)
    a.update(kw)
    return bsa.lib.bsa_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["B"], a["H"],
                                a["Nq"], a["Nk"], a["d"], a["qb"], a["kvb"], a["idx"], a["bias"],
                                a["cnt"], a["L"], a["scale"], a["dq"], a["dk"], a["dv"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), -1), (dict(lse=None), -1), (dict(dk=None), -1), (dict(Nk=0), -1),
    (dict(dv=FAKE + 4096), -1), (dict(dq=FAKE + 8192), -1),
    (dict(scale=float("nan")), -1), (dict(d=96), -2), (dict(kvb=3), -2), (dict(qb=64), -2),
    (dict(dq=FAKE + 4), -4), (dict(do=FAKE + 8), -4), (dict(L=2**28, kvb=128), -7),
])
def test_attn_bwd_rejects_invalid_arguments(bsa, kw, status):
    assert _bwd(bsa, **kw) == status


def _bwd_ws(bsa, ws=FAKE + 65536, ws_bytes=1 << 40, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, B=1, H=1, Nq=300, Nk=300, d=128,
             qb=128, kvb=4, idx=FAKE, bias=None, cnt=FAKE, L=8, scale=0.0, dq=FAKE,
             dk=FAKE + 4096, dv=FAKE + 8192)
    a.update(kw)
    return bsa.lib.bsa_attn_bwd_ws(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["B"],
                                   a["H"], a["Nq"], a["Nk"], a["d"], a["qb"], a["kvb"], a["idx"],
                                   a["bias"], a["cnt"], a["L"], a["scale"], a["dq"], a["dk"],
                                   a["dv"], ws, ws_bytes, None)


def test_attn_bwd_workspace_bytes(bsa):
    """One (b, h) slab: per pair of query blocks, room for a union list of
    2 max_blocks + 3 passes' padding entries (a pass is 128 keys, so
    128 / kv_block blocks, at least one), each with kv_block * 2d fp32
    partial rows; the key-major lists (two arrays of M + 1 ints and two
    slot numbers per union entry, as filled and sorted); the union lists (a
    block and two shifts per entry); three class ends per pair (4 ints).
    Each array is padded to 64 elements."""
    for Nq, Nk, d, kvb, L in [(300, 300, 128, 4, 8), (75600, 75600, 128, 4, 2048),
                              (256, 260, 64, 1, 70), (1000, 1000, 128, 128, 3)]:
        got = bsa.bsa_attn_bwd_workspace_bytes(Nq, Nk, d, L, 128, kvb)
        nqb, M = -(-Nq // 128), -(-Nk // kvb)
        pad = lambda n: -(-n // 64) * 64  # noqa: E731
        pairs, ucap = -(-nqb // 2), 2 * L + 3 * max(1, 128 // kvb)
        want = (pairs * ucap * kvb * 2 * d * 4 + 4 * 2 * pad(M + 1) + 20 * pad(pairs * ucap)
                + 4 * pad(4 * pairs))
        assert got == want
        assert got % 256 == 0
    out = ctypes.c_size_t(0)
    L = bsa.lib
    assert L.bsa_attn_bwd_workspace_bytes(300, 300, 128, 128, 4, 8, None) == -1
    assert L.bsa_attn_bwd_workspace_bytes(0, 300, 128, 128, 4, 8, ctypes.byref(out)) == -1
    assert L.bsa_attn_bwd_workspace_bytes(300, 300, 96, 128, 4, 8, ctypes.byref(out)) == -2
    assert L.bsa_attn_bwd_workspace_bytes(300, 300, 128, 128, 3, 8, ctypes.byref(out)) == -2
    assert L.bsa_attn_bwd_workspace_bytes(2**24, 300, 128, 128, 1, 2**20, ctypes.byref(out)) == -7
    # nQB * max_blocks fits 2^31, the pairs' union entries (with padding) do not
    assert L.bsa_attn_bwd_workspace_bytes(2**23, 300, 128, 128, 4, 2**15 - 1,
                                          ctypes.byref(out)) == -7


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), -1), (dict(dk=None), -1), (dict(dv=FAKE + 4096), -1), (dict(d=96), -2),
    (dict(dq=FAKE + 4), -4), (dict(ws=None), -6), (dict(ws_bytes=4096), -6),
    (dict(ws=FAKE + 65536 + 128), -4), (dict(Nq=2**24, kvb=1, L=2**20), -7),
    (dict(B=2**12, H=2**12, Nk=2**20, kvb=1, Nq=128), -7),
])
def test_attn_bwd_ws_rejects_invalid_arguments(bsa, kw, status):
    """The workspace backward refuses what bsa_attn_bwd refuses, a missing,
    misaligned or too small workspace, and lists whose entry count exceeds
    the index range, before any HIP call."""
    assert _bwd_ws(bsa, **kw) == status


def test_binding_loads_the_library_into_torchs_hip_runtime():
    """Importing the binding in a fresh process maps a single HIP runtime:
    the one torch carries.  (Loaded before torch, libbsa.so would bring in
    /opt/rocm's runtime as a second copy, in which torch's streams and
    memory do not exist.)"""
    import subprocess
    import sys
    code = ("import os, block_sparse_attention_mean_amd\n"
            "m = open(f'/proc/{os.getpid()}/maps').read().splitlines()\n"
            "print(sorted(set(l.split()[-1] for l in m if 'libamdhip64' in l)))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1 and "torch" in libs[0], libs


def test_mfma_probe_rejects_invalid_arguments(bsa):
    """The matrix probe refuses a null or misaligned sink, empty grids or
    rounds and unknown operand modes before any HIP call."""
    L = bsa.lib
    assert bsa.PROBE_RANDOM == 0 and bsa.PROBE_LOW_ENTROPY == 1
    assert L.bsa_mfma_peak_probe(1, 1, 0, None, None, None) == -1
    assert L.bsa_mfma_peak_probe(0, 1, 0, FAKE, None, None) == -1
    assert L.bsa_mfma_peak_probe(1, 0, 1, FAKE, None, None) == -1
    assert L.bsa_mfma_peak_probe(1, 1, 2, FAKE, None, None) == -1
    assert L.bsa_mfma_peak_probe(1, 1, -1, FAKE, None, None) == -1
    assert L.bsa_mfma_peak_probe(1, 1, 0, FAKE + 2, None, None) == -4
