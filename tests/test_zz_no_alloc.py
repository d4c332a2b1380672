"""bsa_basa_plan_noalloc, the allocation-free variant of the BASA list
builder for callers that cannot allocate device memory: its outputs equal
those of bsa_basa_plan (which takes a caller workspace) byte for byte, on two
calls in a row, the second with a smaller problem, so that what the first
call left in the fixed scratch cannot leak into the second.  Sizes whose
scratch exceeds the fixed array are refused on the host."""
import ctypes

import numpy as np
import pytest

from synth import make_qkv

FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced


def test_noalloc_rejects_scratch_beyond_the_fixed_array():
    import block_sparse_attention_mean_amd as bsa
    L = bsa.lib

    def call(H, d=128):
        return L.bsa_basa_plan_noalloc(FAKE, FAKE, FAKE, 1, H, 21, 60, 104, d, 10, 10, 3, 7, 4, 4,
                                       2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    lay = bsa.bsa_basa_layout(21, 60, 104, 128, 10, 10, 4, 4, 2, 4, 1, 64)
    assert lay["workspace"] > 4 << 20
    assert call(64) == -8                   # 64 heads of 66 windows: 4.4 MB of scratch
    assert call(64, d=96) == -2             # ordinary checks still come first
    assert L.bsa_basa_plan_noalloc(None, FAKE, FAKE, 1, 1, 21, 60, 104, 128, 10, 10, 3, 7, 4, 4,
                                   2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert b"scratch" in L.bsa_status_string(-8)


CASES = [
    # (T, Hg, Wg, H, d, wh, ww, dy, dx, ph, pw, topk, kv_block, seed)
    (21, 60, 104, 3, 128, 10, 10, 3, 7, 4, 4, 2, 4, 0),   # the 1664x960 layout, 3 heads
    (2, 20, 26, 2, 64, 10, 10, 5, 1, 2, 2, 3, 4, 1),      # a smaller one, ragged last column
]


@pytest.mark.gpu
def test_noalloc_equals_workspace_variant_on_two_calls():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu as g
    for T, Hg, Wg, H, d, wh, ww, dy, dx, ph, pw, topk, kvb, seed in CASES:
        g.say(f"case noalloc basa plan T={T} Hg={Hg} Wg={Wg} H={H} d={d} w=({wh},{ww}) "
              f"roll=({dy},{dx}) pool=({ph},{pw}) topk={topk} kv_block={kvb}")
        qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=seed)
        q, k, v = g.to_dev_bf16(qb), g.to_dev_bf16(kb), g.to_dev_bf16(vb)
        ref = bsa.bsa_basa_plan(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kvb,
                                want_routes=True)
        # outputs preallocated and filled with garbage, then the allocation-free call
        out = {key: torch.full_like(ref[key], -7) for key in ("idx", "count", "routes")}
        for key in ("qp", "kp", "vp"):
            out[key] = torch.full_like(ref[key], 3.0)
        torch.cuda.synchronize()
        got = bsa.bsa_basa_plan_noalloc(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kvb,
                                        out=out)
        torch.cuda.synchronize()
        for key in ("qp", "kp", "vp", "idx", "count", "routes"):
            assert got[key] is out[key]
            a = got[key].view(torch.int16) if got[key].dtype == torch.bfloat16 else got[key]
            b = ref[key].view(torch.int16) if ref[key].dtype == torch.bfloat16 else ref[key]
            assert torch.equal(a, b), f"{key} differs"
        g.say(f"  equal: qp {tuple(got['qp'].shape)} idx {tuple(got['idx'].shape)} "
              f"routes {got['routes'].flatten()[:6].tolist()}")
