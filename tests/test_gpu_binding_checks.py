"""The Python binding refuses wrongly shaped, typed, placed or laid-out
tensors with ValueError before any launch, so that a caller's mistake never
becomes an out-of-bounds device access.  These tests need device tensors
but launch no kernel."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    return bsa, torch


def _t(torch, shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_attn_fwd_checks(env):
    bsa, torch = env
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    q = _t(torch, (1, 2, 300, 128), bf)
    k = _t(torch, (1, 2, 200, 128), bf)
    idx, cnt = _t(torch, (1, 2, 3, 10), i32), _t(torch, (1, 2, 3), i32)
    bias = _t(torch, (1, 2, 3, 10), f32)
    good = dict(q=q, k=k, v=k, idx=idx, bias=bias, count=cnt)
    bad = [
        dict(k=_t(torch, (1, 2, 200, 64), bf)),           # head dim differs
        dict(k=_t(torch, (1, 3, 200, 128), bf)),          # heads differ
        dict(v=_t(torch, (1, 2, 201, 128), bf)),          # v is not k's shape
        dict(idx=_t(torch, (1, 2, 2, 10), i32)),          # query blocks: 3
        dict(idx=_t(torch, (1, 2, 3, 10), torch.int64)),  # dtype
        dict(bias=_t(torch, (1, 2, 3, 9), f32)),          # list length differs
        dict(count=_t(torch, (1, 2, 4), i32)),
        dict(count=_t(torch, (1, 2, 3), i32).cpu()),      # host tensor
        dict(q=_t(torch, (1, 2, 128, 300), bf).transpose(2, 3)),   # not contiguous
        dict(out=_t(torch, (1, 2, 300, 64), bf)),
        dict(lse=_t(torch, (1, 2, 299), f32)),
    ]
    for b in bad:
        kw = dict(good, **b)
        extra = {x: kw.pop(x) for x in ("out", "lse") if x in kw}
        with pytest.raises(ValueError):
            bsa.bsa_attn_fwd(kw["q"], kw["k"], kw["v"], kw["idx"], kw["bias"], kw["count"],
                             128, 4, **extra)


def test_attn_bwd_checks(env):
    bsa, torch = env
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    q = _t(torch, (1, 1, 256, 64), bf)
    k = _t(torch, (1, 1, 128, 64), bf)
    lse = _t(torch, (1, 1, 256), f32)
    idx, cnt = _t(torch, (1, 1, 2, 4), i32), _t(torch, (1, 1, 2), i32)
    base = dict(q=q, k=k, v=k, out=q, dout=q, lse=lse, idx=idx, bias=None, count=cnt)
    bad = [dict(dout=_t(torch, (1, 1, 255, 64), bf)), dict(lse=_t(torch, (1, 1, 128), f32)),
           dict(out=_t(torch, (1, 1, 256, 64), f32)), dict(v=_t(torch, (1, 1, 129, 64), bf)),
           dict(dk=_t(torch, (1, 1, 256, 64), f32)), dict(dq=_t(torch, (1, 1, 256, 64), bf))]
    names = ("q", "k", "v", "out", "dout", "lse", "idx", "bias", "count")
    for b in bad:
        kw = dict(base, **b)
        extra = {x: kw.pop(x) for x in ("dq", "dk", "dv") if x in kw}
        for fn in (bsa.bsa_attn_bwd, bsa.bsa_attn_bwd_ws):
            with pytest.raises(ValueError):
                fn(*[kw[n] for n in names], 128, 4, **extra)
    # the workspace form: a workspace of the wrong dtype or device is refused
    # by the binding; one smaller than a slab by the library (no launch)
    args = [base[n] for n in names]
    for ws in (_t(torch, (4096,), f32), _t(torch, (4096,), torch.uint8).cpu()):
        with pytest.raises(ValueError):
            bsa.bsa_attn_bwd_ws(*args, 128, 4, workspace=ws)
    need = bsa.bsa_attn_bwd_workspace_bytes(256, 128, 64, 4, 128, 4)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_attn_bwd_ws(*args, 128, 4, workspace=_t(torch, (need - 256,), torch.uint8))
    assert e.value.status == -6


def test_plan_and_select_checks(env):
    bsa, torch = env
    i32, f32 = torch.int32, torch.float32
    S = _t(torch, (1, 2, 3, 100), f32)
    for kw in (dict(idx=_t(torch, (1, 2, 3, 9), i32)), dict(bias=_t(torch, (1, 2, 3, 11), f32)),
               dict(count=_t(torch, (2, 3), i32)), dict(lam=_t(torch, (1, 2, 3), f32)),
               dict(offsets=_t(torch, (5,), torch.int64)), dict(status=_t(torch, (2,), i32)),
               dict(status=_t(torch, (1,), torch.int64))):
        with pytest.raises(ValueError):
            bsa.bsa_sip_plan(S, 10, bsa.PLAN_SIP, **kw)
    q = _t(torch, (1, 2, 256, 128), torch.bfloat16)
    for kw in (dict(scores=_t(torch, (1, 2, 2, 63), f32)),
               dict(centroids=_t(torch, (1, 2, 2, 4, 128), f32), weights=_t(torch, (1, 2, 2, 8), f32)),
               dict(workspace=_t(torch, (16,), f32))):
        with pytest.raises(ValueError):
            bsa.bsa_select_scores(q, q, 128, 4, 8, 1, **kw)
    with pytest.raises(ValueError):
        bsa.bsa_select_scores(q, _t(torch, (1, 2, 255, 128), torch.bfloat16), 128, 4)


def test_basa_and_diag_checks(env):
    bsa, torch = env
    bf, f32 = torch.bfloat16, torch.float32
    q = _t(torch, (1, 1, 2 * 20 * 26, 64), bf)
    with pytest.raises(ValueError):
        bsa.bsa_basa_plan(q, _t(torch, (1, 1, 2 * 20 * 26, 128), bf), q, 2, 20, 26, 10, 10, 0, 0,
                          2, 2, 1)
    with pytest.raises(ValueError):     # the grid holds 1,040 tokens, q 1,039
        bsa.bsa_basa_plan(q[:, :, 1:].contiguous(), q[:, :, 1:].contiguous(),
                          q[:, :, 1:].contiguous(), 2, 20, 26, 10, 10, 0, 0, 2, 2, 1)
    with pytest.raises(ValueError):     # window-major rows differ from the layout's
        bsa.bsa_window_unpermute(q, 2, 20, 26, 10, 10, 0, 0)
    k = _t(torch, (1, 1, 300, 64), bf)
    with pytest.raises(ValueError):
        bsa.bsa_block_mass(q, k, _t(torch, (1, 1, 300), f32))
    with pytest.raises(ValueError):
        bsa.bsa_block_mass(q, k, _t(torch, (1, 1, 1040), f32), mass=_t(torch, (1, 1, 9, 76), f32))
    with pytest.raises(ValueError):
        bsa.bsa_output_error(q, _t(torch, (1, 1, 1040, 32), bf))
    with pytest.raises(ValueError):
        bsa.bsa_output_error(q, q, sums=_t(torch, (1, 2, 2), torch.float64))
