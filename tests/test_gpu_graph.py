"""The whole forward step (bsa_select_scores -> bsa_sip_plan -> bsa_attn_fwd)
and the workspace backward captured once into a HIP graph (torch.cuda.graph)
and replayed: every call of the library is asynchronous on the caller's
stream, with no allocation, memset, copy or synchronisation inside, so a
serving loop can replay the step instead of launching it.  Each replay is
checked against an eager run on the same inputs, with other inputs copied
into the graph's buffers between replays and eager work in between.  The
forward kernels are deterministic, so the forward outputs must match bit
for bit; dK and dV of the workspace backward sum in an order that varies
from run to run (the key-major lists are filled with integer atomics), so
they are compared to fp32 summation-order error, dQ bit for bit."""
import numpy as np
import pytest

from synth import make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_mean_amd as bsa
    from tests import _gpu
    return bsa, _gpu, torch


def test_step_graph_replays(env):
    bsa, g, torch = env
    T, Hg, Wg, H, d, kvb, C, s = 4, 16, 24, 3, 128, 4, 8, 96
    N = T * Hg * Wg
    nqb, M = -(-N // 128), -(-N // kvb)
    g.say(f"case graph step N={N} H={H} budget={s}")
    inputs = []
    for seed in (3, 4):
        qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=seed)
        db, _, _ = make_qkv(T, Hg, Wg, H, d, seed=seed + 10)
        inputs.append(tuple(g.to_dev_bf16(x) for x in (qb, kb, vb, db)))
    dev = torch.device("cuda")
    f32, i32 = torch.float32, torch.int32
    q, k, v, dout = (torch.empty_like(x) for x in inputs[0])
    scores = torch.empty((1, H, nqb, M), dtype=f32, device=dev)
    ws = torch.empty(bsa.bsa_select_workspace_bytes(1, H, N, d, 128, kvb, C), dtype=torch.uint8,
                     device=dev)
    idx = torch.empty((1, H, nqb, s), dtype=i32, device=dev)
    bias = torch.empty((1, H, nqb, s), dtype=f32, device=dev)
    cnt = torch.empty((1, H, nqb), dtype=i32, device=dev)
    status = torch.empty(1, dtype=i32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((1, H, N), dtype=f32, device=dev)
    bws = torch.empty(bsa.bsa_attn_bwd_workspace_bytes(N, N, d, s, 128, kvb) * H,
                      dtype=torch.uint8, device=dev)
    dq = torch.empty((1, H, N, d), dtype=f32, device=dev)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    outs = (scores, idx, bias, cnt, status, out, lse, dq, dk, dv)

    def step():
        bsa.bsa_select_scores(q, k, 128, kvb, C, 1, scores=scores, workspace=ws)
        bsa.bsa_sip_plan(scores, s, bsa.PLAN_SIP, seed=5, idx=idx, bias=bias, count=cnt,
                         status=status)
        bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, out=out, lse=lse)
        bsa.bsa_attn_bwd_ws(q, k, v, out, dout, lse, idx, bias, cnt, 128, kvb, dq=dq, dk=dk,
                            dv=dv, workspace=bws)

    def load(i):
        for dst, src in zip((q, k, v, dout), inputs[i]):
            dst.copy_(src)

    eager = []
    for i in range(2):
        load(i)
        step()
        torch.cuda.synchronize()
        eager.append([x.clone() for x in outs])
        assert int(status.item()) == 0 and int(cnt.min().item()) == s

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    names = ("scores", "idx", "bias", "count", "status", "out", "lse", "dq", "dk", "dv")
    for r, i in enumerate((0, 1, 0, 1)):
        for x in outs:  # eager work that clobbers every output between replays
            x.fill_(-7 if x.dtype == i32 else float("nan"))
        load(i)
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, eager[i]):
            if name in ("dk", "dv"):
                rel = float((got.double() - want.double()).norm() / want.double().norm())
                assert rel <= 1e-5, f"replay {r} ({i}) {name}: rel {rel}"
            else:
                assert torch.equal(got, want), f"replay {r} (inputs {i}): {name} differs"
        g.say(f"  replay {r} (inputs {i}) matches the eager run")


def test_basa_noalloc_graph_replays(env):
    """The BASA step through the allocation-free list builder (its scratch in
    the library's fixed device array, looked up once per device by an eager
    call first), then the attention over the lists and the un-permute,
    captured into one graph and replayed with inputs swapped: every output
    equals an eager run's, byte for byte."""
    bsa, g, torch = env
    T, Hg, Wg, H, d, wh, ww, dy, dx, ph, pw, topk, kvb = 2, 20, 26, 2, 64, 10, 10, 5, 1, 2, 2, 3, 4
    g.say(f"case graph basa noalloc T={T} Hg={Hg} Wg={Wg} H={H} d={d}")
    inputs = [tuple(g.to_dev_bf16(x) for x in make_qkv(T, Hg, Wg, H, d, seed=s)) for s in (5, 6)]
    q, k, v = (torch.empty_like(x) for x in inputs[0])
    lists = bsa.bsa_basa_plan_noalloc(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kvb,
                                      want_routes=True)  # allocates the outputs, looks up scratch
    o = {key: lists[key] for key in ("qp", "kp", "vp", "idx", "count", "routes")}
    out_perm = torch.empty_like(o["qp"])
    out = torch.empty_like(q)

    def step():
        bsa.bsa_basa_plan_noalloc(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kvb, out=o)
        bsa.bsa_attn_fwd(o["qp"], o["kp"], o["vp"], o["idx"], None, o["count"], 128, kvb,
                         out=out_perm)
        bsa.bsa_window_unpermute(out_perm, T, Hg, Wg, wh, ww, dy, dx, out=out)

    outs = (o["qp"], o["kp"], o["vp"], o["idx"], o["count"], o["routes"], out_perm, out)
    eager = []
    for i in range(2):
        for dst, src in zip((q, k, v), inputs[i]):
            dst.copy_(src)
        step()
        torch.cuda.synchronize()
        eager.append([x.clone() for x in outs])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    names = ("qp", "kp", "vp", "idx", "count", "routes", "out_perm", "out")
    for r, i in enumerate((1, 0, 1)):
        for x in outs:
            x.view(torch.int16 if x.dtype == torch.bfloat16 else x.dtype).fill_(-7)
        for dst, src in zip((q, k, v), inputs[i]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, eager[i]):
            a = got.view(torch.int16) if got.dtype == torch.bfloat16 else got
            b = want.view(torch.int16) if want.dtype == torch.bfloat16 else want
            assert torch.equal(a, b), f"replay {r} (inputs {i}): {name} differs"
        g.say(f"  replay {r} (inputs {i}) matches the eager run")
