"""Benchmark of the block-sparse attention forward hot path on one MI355X.

One step = the whole path on one batch of synthetic input already resident
in HBM: bsa_select_scores (pooling, k-means, block scores) -> bsa_sip_plan
(SIP, budget 2048) -> bsa_attn_fwd, at the Wan2.1-14B 720p / 81-frame latent
shape (21 x 45 x 80 = 75,600 tokens, 40 heads, d = 128, KV block 4, 89.16 %
sparse).

Prints ONE JSON line.  ``value`` is the effective attention throughput of the
whole step: 4 d x (valid query, selected valid key) pairs / step time.  The
attention kernel alone, the selector and the planner are reported beside it,
with the roofline of the attention kernel (timed with HIP events on the
stream it runs on) and the CPU oracle on a bounded sample.

With ``--workload basa_1664x960`` the step is instead the BASA-structured
path at the 1664x960 / 81-frame latent (21 x 60 x 104, 12 heads, 10 x 10
windows, 4 x 4 pooled memory, top-2 routing): bsa_basa_plan ->
bsa_attn_fwd -> bsa_window_unpermute, reported the same way
(``basa_1664x960_p2``: 2 x 2 pooling; ``basa_1664x960_w15x26``: 15 x 26
windows).  ``--workload wan13b_480p`` (Wan2.1-1.3B 480p, SIP budget 887),
``hunyuan_720p`` (HunyuanVideo 720p, 118,800 tokens, SIP budget 2272) and
``tiny_2x32x32`` (top-8 of 64-token blocks) time the same step as the
headline at those shapes, under their own metric name and without a
traffic figure (the counter runs cover the headline workload).

With ``--accuracy`` it prints instead one JSON report of the accuracy
diagnostics (block_sparse_attention_mean_amd.accuracy) on the first
``--accuracy-heads`` heads of the workload at its token budget: the oracle
top-k's retained mass against KV block size, the output error of SIP, of an
oracle top-k and of the ablation variants against dense attention, and the
timing of the block-mass kernel.

With ``--curve`` it prints one JSON report of the latency-density curve at
the workload's shape: the selector once, then for SIP budgets from 1 % to
100 % of the KV blocks the plan and the attention times, against two dense
bf16 attentions of the same shape (bsa_attn_fwd over every 128-token block,
and torch's flash SDPA timed in a child process), with the sparse/dense
crossover.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workload wan14b_720p|wan13b_480p|hunyuan_720p|tiny_2x32x32|
                                   basa_1664x960|basa_1664x960_p2|basa_1664x960_w15x26]
       python bench.py --accuracy [--workload wan14b_720p] [--accuracy-heads 40]
       python bench.py --curve [--workload wan14b_720p]
       python bench.py --backward [--workload wan14b_720p]
       python bench.py --mfma-peak

With ``--backward`` it prints one JSON report of the backward at the
workload: the selector's SIP plan, one forward call for the output and its
LSE, then bsa_attn_bwd (atomic adds) and bsa_attn_bwd_ws (partial rows per
union entry of two query blocks' lists, ``--bwd-slabs`` (b, h) slabs of
workspace per pass) timed
with HIP events (warmup + steps), against the algorithmic 10 d flops per
(valid query, listed valid key) pair, and the two results compared.

With ``--mfma-peak`` it prints one JSON report of the bf16 matrix-instruction
throughput probe (bsa_mfma_peak_probe: v_mfma_f32_32x32x16_bf16, the
attention kernel's instruction, from registers) over a sweep of grid sizes,
with random operands and with low-entropy operands: the rate the matrix
units sustain drops with the operands' toggling (the clock falls under the
power).  The benchmark line runs the random-operand probe after the timed
region and states the attention kernel's fraction of that measured rate
beside the fraction of the published peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, published spec
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan14b_720p_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_mean_amd", "csrc", "attn_fwd.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="wan14b_720p")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-heads", type=int, default=3,
                   help="whole heads of the workload in the oracle sample")
    p.add_argument("--accuracy", action="store_true",
                   help="print the accuracy diagnostics report instead of the benchmark line")
    p.add_argument("--accuracy-heads", type=int, default=40)
    p.add_argument("--curve", action="store_true",
                   help="print the latency-density curve report instead of the benchmark line")
    p.add_argument("--dense-sdpa", action="store_true",
                   help="(child of --curve) time torch's flash SDPA at the workload's shape")
    p.add_argument("--reps", type=int, default=3)
    p.add_argument("--backward", action="store_true",
                   help="print the backward-pass report instead of the benchmark line")
    p.add_argument("--bwd-slabs", type=int, default=8,
                   help="(b, h) slabs of workspace per pass of bsa_attn_bwd_ws")
    p.add_argument("--mfma-peak", action="store_true",
                   help="print the matrix-instruction throughput report instead of the line")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="after timing, run one device copy of this size (counter calibration)")
    return p.parse_args()


def attn_build_sha():
    """Hash of the attention kernel's code (its source without comments and
    blank lines) and its per-file build flags: what the committed counter
    runs must have been taken on."""
    from block_sparse_attention_mean_amd.build import FILE_FLAGS
    code = re.sub(r"//[^\n]*", "", open(ATTN_SRC).read())
    code = "\n".join(ln.rstrip() for ln in code.splitlines() if ln.strip())
    h = hashlib.sha256(code.encode())
    h.update(" ".join(FILE_FLAGS.get("attn_fwd.hip", [])).encode())
    return h.hexdigest()


def traffic_for_current_kernel():
    """HBM bytes per attention launch from committed counter runs, if they
    were taken on the current kernel build; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_build_sha256") != attn_build_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def attn_kernel_name(d, kv_block, Nk):
    """The attention instance a call launches: group shifts when every wave
    load (4 rows at d = 128, 8 at d = 64) lies inside one KV block, with the
    Nk-crossing checks when Nk is not a whole number of wave loads; the
    half-load variant when KV blocks are half a load and Nk a whole number
    of blocks (below 4 GiB of rows)."""
    rows = 4 if d == 128 else 8
    if 2 * kv_block == rows and Nk % kv_block == 0 and Nk * d * 2 <= 1 << 32:
        return f"bsa::attn_fwd_kernel<{d}, true, false, true>"
    quad = kv_block >= rows
    part = quad and Nk % rows != 0
    return f"bsa::attn_fwd_kernel<{d}, {str(quad).lower()}, {str(part).lower()}, false>"


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def cpu_baseline(c, seed, heads, one_thread_heads=1):
    """The oracle (as it stands) on whole heads 0..heads-1 of the workload:
    pooling, k-means, scores, plan (SIP, or top-k where the workload says
    so) and attention of every query block, on all the host's BLAS threads;
    then the same on heads 0..one_thread_heads-1 with BLAS limited to one
    thread.  Returns effective TFLOP/s (same definition as the GPU value),
    seconds per head, and seconds per head times the workload's head count
    (an extrapolation, labelled as such)."""
    rec = _oracle_run(c, seed, heads)
    rec.update({
        "kind": "oracle", "cores": rec.pop("threads"),
        "sample": (f"heads 0..{heads - 1} of {c['name']} (all query blocks): pooling, k-means, "
                   f"scores, {'top-k' if c.get('mode') == 'topk' else 'SIP'} plan and attention, "
                   f"fp64 numpy (k-means in its stated fp32 order)"),
        "seconds_per_head": round(rec["seconds"] / heads, 3),
        "extrapolated_seconds_all_heads": round(rec["seconds"] / heads * c["H"], 1),
        "extrapolation": f"seconds per head x {c['H']} heads (not measured)",
        "host_cpus": os.cpu_count(), "host_cpu_model": host_cpu_model(),
    })
    if one_thread_heads:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            one = _oracle_run(c, seed, one_thread_heads)
        rec["one_thread"] = {
            "value": one["value"], "unit": "TFLOP/s", "cores": one["threads"],
            "sample": f"heads 0..{one_thread_heads - 1} of {c['name']}, the same stages",
            "seconds": one["seconds"], "stage_seconds": one["stage_seconds"],
            "seconds_per_head": round(one["seconds"] / one_thread_heads, 3),
            "extrapolated_seconds_all_heads": round(one["seconds"] / one_thread_heads * c["H"], 1),
        }
    return rec


def _oracle_run(c, seed, heads):
    import numpy as np
    from oracle import attn as oat
    from oracle import plan as opl
    from oracle import select as osel
    from synth import bf16_bits_to_f32, bf16_bits_to_f64, head_qkv
    threads = blas_threads()
    st = {"select": 0.0, "plan": 0.0, "attn": 0.0}
    flops = 0.0
    for h in range(heads):
        qb, kb, vb = head_qkv(c["T"], c["Hg"], c["Wg"], c["d"], seed, h)
        q32 = bf16_bits_to_f32(qb)
        q, k, v = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
        N, d, kvb, s = q.shape[0], c["d"], c["kv_block"], c["budget"]
        nqb = -(-N // 128)
        t0 = time.perf_counter()
        kbar = osel.pool_keys(k, kvb)
        mu, w = osel.kmeans_head(q32, 128, c["n_clusters"], c["kmeans_iters"])
        S = osel.scores_from_centroids(mu, w, kbar)
        t1 = time.perf_counter()
        mode = opl.TOPK if c.get("mode") == "topk" else opl.SIP
        idx, bias, cnt, _ = opl.plan(S, s, mode, seed=seed, row_base=h * nqb)
        t2 = time.perf_counter()
        oat.attn_fwd(q, k, v, 128, kvb, idx, bias, cnt)
        t3 = time.perf_counter()
        st["select"] += t1 - t0
        st["plan"] += t2 - t1
        st["attn"] += t3 - t2
        flops += sum(4.0 * d * min(128, N - 128 * i) * int(cnt[i]) * kvb for i in range(nqb))
    total = sum(st.values())
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "threads": int(threads),
            "seconds": round(total, 3),
            "stage_seconds": {k2: round(v2, 3) for k2, v2 in st.items()}}


def basa_window_rows(T, Hg, Wg, wh, ww):
    """(first padded row, token count) of every window, window-major order."""
    nwy, nwx = -(-Hg // wh), -(-Wg // ww)
    out, off = [], 0
    for a in range(nwy):
        for b in range(nwx):
            n = T * (min(Hg, (a + 1) * wh) - a * wh) * (min(Wg, (b + 1) * ww) - b * ww)
            out.append((off, n))
            off += -(-n // 128) * 128
    return out, off


def basa_cpu_baseline(c, seed, heads):
    """The oracle's definition-based BASA attention of whole heads 0..heads-1
    (window routing and every window's output rows), in the same TFLOP/s
    unit."""
    import numpy as np
    from oracle import basa as obasa
    from synth import bf16_bits_to_f32, head_qkv
    threads = blas_threads()
    members = obasa.window_members(c["T"], c["Hg"], c["Wg"], c["wh"], c["ww"], c["dy"], c["dx"])
    npool = c["T"] * -(-c["Hg"] // c["ph"]) * -(-c["Wg"] // c["pw"])
    sec, flops = 0.0, 0.0
    for h in range(heads):
        qb, kb, vb = head_qkv(c["T"], c["Hg"], c["Wg"], c["d"], seed, h)
        t0 = time.perf_counter()
        routes = obasa.route(bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), members, c["topk"])
        obasa.basa_attn(qb, kb, vb, c["T"], c["Hg"], c["Wg"], c["wh"], c["ww"], c["dy"], c["dx"],
                        c["ph"], c["pw"], c["topk"], routes=routes)
        sec += time.perf_counter() - t0
        flops += sum(4.0 * c["d"] * len(members[w]) *
                     (len(members[w]) + sum(len(members[j]) for j in routes[w]) + npool)
                     for w in range(len(members)))
    return {
        "value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"heads 0..{heads - 1} of {c['name']}, all {len(members)} windows: routing and "
                   f"attention, fp64 numpy (routing in its stated fp32 order)"),
        "seconds": round(sec, 3), "seconds_per_head": round(sec / heads, 3),
        "extrapolated_seconds_all_heads": round(sec / heads * c["H"], 1),
        "extrapolation": f"seconds per head x {c['H']} heads (not measured)",
        "host_cpus": os.cpu_count(), "host_cpu_model": host_cpu_model(),
    }


def run_basa(args):
    import numpy as np
    import torch
    import block_sparse_attention_mean_amd as bsa
    from synth import CONFIGS, make_qkv

    c = dict(CONFIGS[args.workload])
    c["name"] = args.workload
    T, Hg, Wg, H, d, kvb = c["T"], c["Hg"], c["Wg"], c["H"], c["d"], c["kv_block"]
    wh, ww, dy, dx, ph, pw, topk = (c[x] for x in ("wh", "ww", "dy", "dx", "ph", "pw", "topk"))
    N = T * Hg * Wg
    dev = torch.device("cuda:0")
    log(f"[bench] generating {args.workload}: H={H} N={N} d={d}")
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=args.seed, workers=min(16, os.cpu_count() or 1))
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    del qb, kb, vb
    lay = bsa.bsa_basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kvb, 1, H)
    nq, nk, mb = lay["Nq_pad"], lay["Nk"], lay["max_blocks"]
    nqb = nq // 128
    qp = torch.empty((1, H, nq, d), dtype=torch.bfloat16, device=dev)
    kp = torch.empty((1, H, nk, d), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    idx = torch.empty((1, H, nqb, mb), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, H, nqb), dtype=torch.int32, device=dev)
    ws = torch.empty(max(lay["workspace"], 256), dtype=torch.uint8, device=dev)
    outp = torch.empty_like(qp)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    L = bsa.lib
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        if marks is not None:
            marks[0].record(stream)
        bsa._check(L.bsa_basa_plan(q.data_ptr(), k.data_ptr(), v.data_ptr(), 1, H, T, Hg, Wg, d,
                                   wh, ww, dy, dx, ph, pw, topk, kvb, qp.data_ptr(), kp.data_ptr(),
                                   vp.data_ptr(), idx.data_ptr(), cnt.data_ptr(), None,
                                   ws.data_ptr(), ws.numel(), st), "bsa_basa_plan")
        if marks is not None:
            marks[1].record(stream)
        bsa._check(L.bsa_attn_fwd(qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), 1, H, nq, nk, d,
                                  128, kvb, idx.data_ptr(), None, cnt.data_ptr(), mb, 0.0,
                                  outp.data_ptr(), None, st), "bsa_attn_fwd")
        if marks is not None:
            marks[2].record(stream)
        bsa._check(L.bsa_window_unpermute(outp.data_ptr(), out.data_ptr(), 1, H, T, Hg, Wg, d, wh,
                                          ww, dy, dx, st), "bsa_window_unpermute")
        if marks is not None:
            marks[3].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks = [[ev() for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    g0, g1 = ev(), ev()
    g0.record(stream)
    for i in range(args.steps):
        step(marks[i])
    g1.record(stream)
    torch.cuda.synchronize()
    ms_step = g0.elapsed_time(g1) / args.steps
    prep = float(np.median([m[0].elapsed_time(m[1]) for m in marks]))
    att = float(np.median([m[1].elapsed_time(m[2]) for m in marks]))
    unp = float(np.median([m[2].elapsed_time(m[3]) for m in marks]))
    # algorithmic work: real (unpadded) queries x valid keys of their lists
    wins, _ = basa_window_rows(T, Hg, Wg, wh, ww)
    qvalid = np.zeros(nqb, np.int64)
    for off, n in wins:
        for i in range(off // 128, (off + n + 127) // 128):
            qvalid[i] = min(128, off + n - 128 * i)
    idx_h = idx.cpu().numpy().astype(np.int64)
    cnt_h = cnt.cpu().numpy().astype(np.int64)
    e = np.arange(mb)[None, None, None, :]
    keys = np.where(e < cnt_h[..., None], np.minimum(kvb, nk - idx_h * kvb), 0).sum(axis=-1)
    flops = 4.0 * d * float((keys * qvalid[None, None, :]).sum())
    if not torch.isfinite(out.float()).all():
        raise SystemExit("non-finite attention output")
    attn_tf = flops / att / 1e9
    npool = T * -(-Hg // ph) * -(-Wg // pw)
    dense_keys = N
    rec = {
        "metric": "BASA-structured block-sparse attention effective TFLOP/s, 1664x960x81 latent",
        "value": round(flops / ms_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: latent {T}x{Hg}x{Wg} = {N} tokens, B=1, H={H}, d={d}, "
                        f"windows {wh}x{ww} rolled by ({dy},{dx}), pooled {ph}x{pw} ({npool} tokens), "
                        f"top-{topk} routing, KV block {kvb}",
            "B": 1, "H": H, "N": N, "d": d, "kv_block": kvb, "Nq_pad": nq, "Nk": nk,
            "max_blocks": mb, "sparsity": round(1 - float(keys.mean()) / dense_keys, 5),
            "seed": args.seed,
            "step": "bsa_basa_plan + bsa_attn_fwd + bsa_window_unpermute",
        },
        "attn_ms_per_call": round(att, 4),
        "attn_tflops": round(attn_tf, 2),
        "basa_plan_ms": round(prep, 4),
        "unpermute_ms": round(unp, 4),
        "attn_flop_per_call": flops,
        "roofline": {
            "kernel": attn_kernel_name(d, kvb, nk),
            "bound": "mfma",
            "achieved": round(attn_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }
    # context, outside the timed step: dense attention of the same raster-order
    # Q/K/V (this library over every 128-token block, no bias)
    del qp, kp, vp, outp, idx, ws
    didx, dcnt = bsa.dense_plan(1, H, N, N, 128, device=dev)
    dense_ms = _time(lambda: bsa.bsa_attn_fwd(q, k, v, didx, None, dcnt, 128, 128, out=out), 2)
    rec["dense_attn_ms"] = round(dense_ms, 4)
    rec["speedup_vs_dense_attn"] = round(dense_ms / ms_step, 3)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        rec["cpu_baseline"] = basa_cpu_baseline(c, args.seed, 2)
    print(json.dumps(rec), flush=True)


def run_accuracy(args):
    """Accuracy diagnostics of the workload's plans (see the module docstring)."""
    import numpy as np
    import torch
    import block_sparse_attention_mean_amd as bsa
    from block_sparse_attention_mean_amd import accuracy as acc
    from synth import CONFIGS, make_qkv

    c = CONFIGS[args.workload]
    T, Hg, Wg, d = c["T"], c["Hg"], c["Wg"], c["d"]
    H = min(args.accuracy_heads, c["H"])
    N = T * Hg * Wg
    tokens = c["budget"] * c["kv_block"]
    dev = torch.device("cuda:0")
    log(f"[accuracy] generating {args.workload}: heads 0..{H - 1}, N={N}")
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=args.seed, workers=min(16, os.cpu_count() or 1))
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    del qb, kb, vb
    log("[accuracy] dense reference")
    ref, lse = acc.dense_reference(q, k, v)
    torch.cuda.synchronize()

    # block-mass kernel timing (4-token blocks), HIP events on its stream
    stream = torch.cuda.current_stream()
    mass = bsa.bsa_block_mass(q, k, lse, 128, 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        bsa.bsa_block_mass(q, k, lse, 128, 4, mass=mass)
    e1.record(stream)
    torch.cuda.synchronize()
    mass_ms = e0.elapsed_time(e1) / reps
    mass_tf = 2.0 * d * N * N * H / mass_ms / 1e9
    row_sums = mass.double().sum(dim=-1)
    row_dev = float((row_sums - 1).abs().max())
    del mass

    log("[accuracy] oracle top-k curve")
    curve = acc.oracle_topk_curve(q, k, lse, tokens)
    log("[accuracy] variants")
    var = acc.variants(q, k, v, ref, lse, tokens, seed=args.seed, n_clusters=c["n_clusters"],
                       kmeans_iters=c["kmeans_iters"])
    mean = lambda a: round(float(np.mean(a)), 5)  # noqa: E731
    rep = {
        "report": "accuracy",
        "workload": f"{args.workload}: latent {T}x{Hg}x{Wg} = {N} tokens, heads 0..{H - 1}, "
                    f"d={d}, token budget {tokens} ({100 * tokens / N:.2f} % of the keys)",
        "data": "synthetic",
        "seed": args.seed,
        "oracle_topk_retained_mass": {str(b): mean(r) for b, r in curve.items()},
        "variants": {n: {"error": mean(r["error"]),
                         "error_per_head": [round(float(x), 5) for x in np.ravel(r["error"])],
                         **({"retained_mass": mean(r["retained_mass"])}
                            if "retained_mass" in r else {})}
                     for n, r in var.items()},
        "sip_error_vs_oracle_topk": round(float(np.mean(var["ibcs_sip"]["error"])
                                                / np.mean(var["oracle_topk"]["error"])), 4),
        "block_mass": {"kernel": "bsa::block_mass_kernel<128>", "kv_block": 4,
                       "ms_per_call": round(mass_ms, 4), "achieved": round(mass_tf, 2),
                       "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(mass_tf / PEAK_BF16_TFLOPS, 4), "bound": "mfma",
                       "max_row_sum_deviation": row_dev},
    }
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rep["copy_calib_bytes"] = n
    print(json.dumps(rep), flush=True)


CURVE_DENSITIES = (0.01, 0.02, 0.05, None, 0.2, 0.3, 0.5, 0.75, 1.0)   # None: the workload's


def _inputs(args, c, H=None):
    import numpy as np
    import torch
    from synth import make_qkv
    H = c["H"] if H is None else H
    qb, kb, vb = make_qkv(c["T"], c["Hg"], c["Wg"], H, c["d"], seed=args.seed,
                          workers=min(16, os.cpu_count() or 1))
    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    return to_dev(qb), to_dev(kb), to_dev(vb)


def _time(fn, reps, warmup=1):
    """Mean ms per call over reps calls (HIP events on the current stream)."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def mfma_peak(workgroups, iters=2000, reps=3, operands=0):
    """Best rate of the matrix-instruction probe over `reps` timed calls
    (TFLOP/s), and the ms of one call; operands 0 = random, 1 = low
    entropy."""
    import torch
    import block_sparse_attention_mean_amd as bsa
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops = bsa.bsa_mfma_peak_probe(workgroups, iters, sink, operands)      # warmup
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bsa.bsa_mfma_peak_probe(workgroups, iters, sink, operands)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return flops / best / 1e9, best


# The probe holds 3 waves per SIMD (about 150 registers each): 768
# workgroups of 4 waves fill the chip once; 3072 run four such rounds.
PEAK_PROBE_GRID = 3072
PEAK_PROBE_ITERS = 4000
PROBE_RESIDENT_WAVES = 3


def run_mfma_peak(args):
    """Throughput of v_mfma_f32_32x32x16_bf16 over grid sizes and operand
    modes (see the module docstring)."""
    pts = []
    for mode, name in ((0, "random"), (1, "low entropy")):
        for wg in (256, 512, 768, PEAK_PROBE_GRID):
            tf, ms = mfma_peak(wg, PEAK_PROBE_ITERS, reps=args.reps, operands=mode)
            pts.append({"operands": name, "workgroups": wg,
                        "resident_waves_per_simd": min(PROBE_RESIDENT_WAVES, wg * 4 // 1024),
                        "ms": round(ms, 4), "tflops": round(tf, 2),
                        "frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4)})
            log(f"[mfma-peak] {pts[-1]}")
    best = {n: max(p["tflops"] for p in pts if p["operands"] == n) for n in ("random", "low entropy")}
    rep = {"report": "mfma peak", "kernel": "bsa::mfma_peak_kernel",
           "instruction": "v_mfma_f32_32x32x16_bf16 (32768 flops), 8 independent chains per wave, "
                          "operands in registers",
           "operands": {"random": "bf16 in +-[1/4, 4), random sign and mantissa, three sets that "
                                  "consecutive instructions alternate between",
                        "low entropy": "a few small values with short mantissas, fixed per lane"},
           "iters": PEAK_PROBE_ITERS, "reps": args.reps, "peak_spec": PEAK_BF16_TFLOPS, "points": pts,
           "best_tflops": best}
    print(json.dumps(rep), flush=True)


def run_dense_sdpa(args):
    """torch flash SDPA (no math fallback) at the workload's shape."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from synth import CONFIGS
    c = CONFIGS[args.workload]
    q, k, v = _inputs(args, c)
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
        f = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v)  # noqa: E731
        ms = _time(f, args.reps)
    print(json.dumps({"sdpa_ms": ms}), flush=True)


def run_backward(args):
    """Backward of the sparse attention at the workload (see the module docstring)."""
    import numpy as np
    import torch
    import block_sparse_attention_mean_amd as bsa
    from synth import CONFIGS

    c = CONFIGS[args.workload]
    T, Hg, Wg, H, d, kvb, C = c["T"], c["Hg"], c["Wg"], c["H"], c["d"], c["kv_block"], c["n_clusters"]
    N, s = T * Hg * Wg, c["budget"]
    nqb = -(-N // 128)
    log(f"[backward] generating {args.workload}: H={H} N={N}")
    q, k, v = _inputs(args, c)
    g = torch.Generator(device="cpu").manual_seed(args.seed + 1)
    dout = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(q.device)
    S, _, _ = bsa.bsa_select_scores(q, k, 128, kvb, C, c["kmeans_iters"])
    idx, bias, cnt, _ = bsa.bsa_sip_plan(S, s, bsa.PLAN_SIP, seed=args.seed)
    del S
    out, lse = bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, want_lse=True)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    f = lambda: bsa.bsa_attn_bwd(q, k, v, out, dout, lse, idx, bias, cnt, 128, kvb,  # noqa: E731
                                 dq=dq, dk=dk, dv=dv)
    fwd_ms = _time(lambda: bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, out=out),
                   args.steps, args.warmup)
    bwd_ms = _time(f, args.steps, args.warmup)
    ch = cnt.cpu().numpy().astype(np.int64)
    rows = np.minimum(128, N - 128 * np.arange(nqb))
    pairs = float((ch[0] * kvb * rows[None, :]).sum())
    for t in (dq, dk, dv):
        if not torch.isfinite(t).all():
            raise SystemExit("non-finite gradient")
    # the workspace variant: partial rows per union entry, summed per KV block
    slab = bsa.bsa_attn_bwd_workspace_bytes(N, N, d, s, 128, kvb)
    nslab = max(1, min(args.bwd_slabs, H))
    log(f"[backward] workspace variant: {nslab} slabs of {slab / 2**30:.2f} GiB per pass")
    ws = torch.empty(slab * nslab, dtype=torch.uint8, device=q.device)
    wq, wk, wv = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    fw = lambda: bsa.bsa_attn_bwd_ws(q, k, v, out, dout, lse, idx, bias, cnt, 128, kvb,  # noqa: E731
                                     dq=wq, dk=wk, dv=wv, workspace=ws)
    ws_ms = _time(fw, args.steps, args.warmup)
    for t in (wq, wk, wv):
        if not torch.isfinite(t).all():
            raise SystemExit("non-finite gradient (workspace variant)")
    diff = {n: float(((a.double() - b.double()).norm() / a.double().norm()).item())
            for n, a, b in (("dq", dq, wq), ("dk", dk, wk), ("dv", dv, wv))}
    # partial rows the workspace form stores: one per entry of the union of
    # the lists of query blocks 2m and 2m + 1, against one per list entry
    ih = idx.cpu().numpy()[0]
    listed = union = 0
    for h in range(H):
        for m in range(0, nqb, 2):
            a_ = ih[h, m, : ch[0, h, m]]
            b_ = ih[h, m + 1, : ch[0, h, m + 1]] if m + 1 < nqb else a_[:0]
            listed += a_.size + b_.size
            union += np.union1d(a_, b_).size
    del ws
    flop = 10.0 * d * pairs
    tf, tfw = flop / bwd_ms / 1e9, flop / ws_ms / 1e9
    rep = {
        "report": "backward",
        "workload": f"{args.workload}: latent {T}x{Hg}x{Wg} = {N} tokens, B=1, H={H}, d={d}, "
                    f"KV block {kvb}, SIP budget {s}",
        "data": "synthetic", "seed": args.seed, "steps": args.steps, "warmup": args.warmup,
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "bwd_over_fwd": round(bwd_ms / fwd_ms, 3),
        "bwd_ws_ms": round(ws_ms, 4), "bwd_ws_over_fwd": round(ws_ms / fwd_ms, 3),
        "bwd_ws_slabs_per_pass": nslab, "bwd_ws_bytes": slab * nslab,
        "ws_vs_atomic_rel_fro": {n: float(f"{x:.3e}") for n, x in diff.items()},
        "ws_partial_rows_per_list_entry": round(union / max(listed, 1), 4),
        "bwd_flop_per_call": flop,
        "roofline": {"kernel": "bsa_attn_bwd (zero + dq + dkdv kernels)", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
        "roofline_ws": {"kernel": "bsa_attn_bwd_ws (dq + key-major lists + dkdv partial rows + "
                                  "per-block sum)", "bound": "mfma",
                        "achieved": round(tfw, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tfw / PEAK_BF16_TFLOPS, 4)},
    }
    print(json.dumps(rep), flush=True)


def run_curve(args):
    """Latency-density curve of the sparse path against dense attention."""
    import subprocess
    import numpy as np
    import torch
    import block_sparse_attention_mean_amd as bsa
    from synth import CONFIGS

    c = CONFIGS[args.workload]
    T, Hg, Wg, H, d, kvb, C = c["T"], c["Hg"], c["Wg"], c["H"], c["d"], c["kv_block"], c["n_clusters"]
    N = T * Hg * Wg
    M, nqb = -(-N // kvb), -(-N // 128)
    rows = np.minimum(128, N - 128 * np.arange(nqb))
    log(f"[curve] generating {args.workload}: H={H} N={N}")
    q, k, v = _inputs(args, c)
    S = torch.empty((1, H, nqb, M), dtype=torch.float32, device=q.device)
    sel_ms = _time(lambda: bsa.bsa_select_scores(q, k, 128, kvb, C, c["kmeans_iters"], scores=S),
                   args.reps)
    points = []
    for f in CURVE_DENSITIES:
        s = c["budget"] if f is None else max(1, min(M, int(round(f * M))))
        log(f"[curve] budget {s} of {M}")
        idx = torch.empty((1, H, nqb, s), dtype=torch.int32, device=q.device)
        bias = torch.empty((1, H, nqb, s), dtype=torch.float32, device=q.device)
        cnt = torch.empty((1, H, nqb), dtype=torch.int32, device=q.device)
        plan = lambda: bsa.bsa_sip_plan(S, s, bsa.PLAN_SIP, seed=args.seed, idx=idx, bias=bias,  # noqa: E731
                                        count=cnt)
        plan_ms = _time(plan, args.reps)
        out = torch.empty_like(q)
        attn_ms = _time(lambda: bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, out=out),
                        args.reps)
        ch = cnt.cpu().numpy().astype(np.int64)
        flops = 4.0 * d * float((ch[0] * kvb * rows[None, :]).sum())
        points.append({"budget": s, "density": round(float(ch.sum()) / (H * nqb * M), 5),
                       "plan_ms": round(plan_ms, 4), "attn_ms": round(attn_ms, 4),
                       "step_ms": round(sel_ms + plan_ms + attn_ms, 4),
                       "attn_tflops": round(flops / attn_ms / 1e9, 2)})
        del idx, bias, cnt, out
    dflops = 4.0 * d * N * N * H
    didx, dcnt = bsa.dense_plan(1, H, N, N, 128, device=q.device)
    dout = torch.empty_like(q)
    dense_ms = _time(lambda: bsa.bsa_attn_fwd(q, k, v, didx, None, dcnt, 128, 128, out=dout),
                     args.reps)
    del q, k, v, S, didx, dout
    torch.cuda.empty_cache()
    log("[curve] torch flash SDPA in a child process")
    sdpa_ms = None
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--dense-sdpa", "--workload",
                            args.workload, "--seed", str(args.seed), "--reps", str(args.reps)],
                           capture_output=True, text=True, timeout=600)
        if r.returncode == 0:
            sdpa_ms = json.loads(r.stdout.strip().splitlines()[-1])["sdpa_ms"]
        else:
            log(f"[curve] SDPA child failed (rc {r.returncode}): {r.stderr[-400:]}")
    except Exception as e:  # noqa: BLE001
        log(f"[curve] SDPA child failed: {e}")
    for p in points:
        p["r_vs_dense_bsa"] = round(p["attn_ms"] / dense_ms, 4)
        if sdpa_ms:
            p["r_vs_sdpa"] = round(p["attn_ms"] / sdpa_ms, 4)

    def crossover(key, ref):
        xs = [p["density"] for p in points]
        ys = [p[key] - ref for p in points]
        for i in range(1, len(xs)):
            if ys[i - 1] < 0 <= ys[i]:
                return round(xs[i - 1] + (xs[i] - xs[i - 1]) * -ys[i - 1] / (ys[i] - ys[i - 1]), 4)
        return None if ys[0] >= 0 else 1.0
    best = min(x for x in (dense_ms, sdpa_ms) if x)
    rep = {
        "report": "latency-density curve",
        "workload": f"{args.workload}: latent {T}x{Hg}x{Wg} = {N} tokens, B=1, H={H}, d={d}, "
                    f"KV block {kvb}, SIP plans of the selector's scores",
        "data": "synthetic", "seed": args.seed, "reps": args.reps,
        "select_ms": round(sel_ms, 4),
        "dense_bsa_ms": round(dense_ms, 4),
        "dense_bsa_tflops": round(dflops / dense_ms / 1e9, 2),
        "dense_sdpa_ms": round(sdpa_ms, 4) if sdpa_ms else None,
        "dense_sdpa_tflops": round(dflops / sdpa_ms / 1e9, 2) if sdpa_ms else None,
        "points": points,
        "crossover_density_attn_vs_best_dense": crossover("attn_ms", best),
        "crossover_density_step_vs_best_dense": crossover("step_ms", best),
    }
    print(json.dumps(rep), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is built and "
              "measured on a single MI355X; heads shard across GPUs with no communication.",
              file=sys.stderr)
        sys.exit(2)
    if args.accuracy:
        return run_accuracy(args)
    if args.dense_sdpa:
        return run_dense_sdpa(args)
    if args.curve:
        return run_curve(args)
    if args.backward:
        return run_backward(args)
    if args.mfma_peak:
        return run_mfma_peak(args)
    if args.workload.startswith("basa"):
        return run_basa(args)
    import numpy as np
    import torch
    import block_sparse_attention_mean_amd as bsa
    from synth import CONFIGS, make_qkv

    c = dict(CONFIGS[args.workload])
    c["name"] = args.workload
    T, Hg, Wg, H, d = c["T"], c["Hg"], c["Wg"], c["H"], c["d"]
    N, kvb, s, C = T * Hg * Wg, c["kv_block"], c["budget"], c["n_clusters"]
    M, nqb = -(-N // kvb), -(-N // 128)
    dev = torch.device("cuda:0")

    log(f"[bench] generating {args.workload}: H={H} N={N} d={d}")
    t0 = time.time()
    qb, kb, vb = make_qkv(T, Hg, Wg, H, d, seed=args.seed, workers=min(16, os.cpu_count() or 1))
    log(f"[bench] inputs drawn in {time.time() - t0:.1f}s")
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    del qb, kb, vb

    ws_bytes = bsa.bsa_select_workspace_bytes(1, H, N, d, 128, kvb, C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scores = torch.empty((1, H, nqb, M), dtype=torch.float32, device=dev)
    idx = torch.empty((1, H, nqb, s), dtype=torch.int32, device=dev)
    bias = torch.empty((1, H, nqb, s), dtype=torch.float32, device=dev)
    cnt = torch.empty((1, H, nqb), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    mode = bsa.PLAN_TOPK if c.get("mode") == "topk" else bsa.PLAN_SIP
    headline = args.workload == "wan14b_720p"

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        if marks is not None:
            marks[0].record(stream)
        bsa.bsa_select_scores(q, k, 128, kvb, C, c["kmeans_iters"], scores=scores, workspace=ws)
        if marks is not None:
            marks[1].record(stream)
        bsa.bsa_sip_plan(scores, s, mode, seed=args.seed, idx=idx, bias=bias, count=cnt)
        if marks is not None:
            marks[2].record(stream)
        bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, out=out)
        if marks is not None:
            marks[3].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks = [[ev() for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    g0, g1 = ev(), ev()
    g0.record(stream)
    for i in range(args.steps):
        step(marks[i])
    g1.record(stream)
    torch.cuda.synchronize()
    ms_step = g0.elapsed_time(g1) / args.steps
    sel = [m[0].elapsed_time(m[1]) for m in marks]
    pln = [m[1].elapsed_time(m[2]) for m in marks]
    att = [m[2].elapsed_time(m[3]) for m in marks]

    # algorithmic attention work of this plan (valid queries x selected valid keys)
    cnt_h = cnt.cpu().numpy().astype(np.int64)
    if (cnt_h != s).any():
        raise SystemExit(f"plan check failed: counts {np.unique(cnt_h)}")
    rows = np.minimum(128, N - 128 * np.arange(nqb))
    # every drawn block is a full 4-token block except a block past N (none for these shapes)
    flops = 4.0 * d * float((cnt_h[0] * kvb * rows[None, :]).sum())
    if not torch.isfinite(out.float()).all():
        raise SystemExit("non-finite attention output")
    attn_ms = float(np.median(att))
    attn_tf = flops / attn_ms / 1e9
    value = flops / ms_step / 1e9
    traffic = traffic_for_current_kernel() if headline else None
    gathered = float(cnt_h.sum() * kvb * d * 2 * 2)
    rec = {
        "metric": ("block-sparse attn ms/call + effective TFLOP/s at Wan-14B 720p shape, 89% sparse"
                   if headline else f"block-sparse attn effective TFLOP/s, {args.workload}"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: latent {T}x{Hg}x{Wg} = {N} tokens, B=1, H={H}, d={d}, "
                        f"query block 128, KV block {kvb}, {C} clusters / {c['kmeans_iters']} "
                        f"k-means iteration, {'top-k' if mode == bsa.PLAN_TOPK else 'SIP'} "
                        f"budget {s} of {M} blocks",
            "B": 1, "H": H, "N": N, "d": d, "kv_block": kvb, "budget": s,
            "sparsity": round(1 - s / M, 5), "seed": args.seed,
            "step": "bsa_select_scores + bsa_sip_plan + bsa_attn_fwd",
        },
        "attn_ms_per_call": round(attn_ms, 4),
        "attn_ms_mean": round(float(np.mean(att)), 4),
        "attn_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(att, [10, 50, 90])],
        "step_ms_p10_p50_p90": [round(float(x), 4) for x in
                                np.percentile([m[0].elapsed_time(m[3]) for m in marks], [10, 50, 90])],
        "attn_tflops": round(attn_tf, 2),
        "select_ms": round(float(np.mean(sel)), 4),
        "plan_ms": round(float(np.mean(pln)), 4),
        "attn_flop_per_call": flops,
        "roofline": {
            "kernel": attn_kernel_name(d, kvb, N),
            "bound": "mfma",
            "achieved": round(attn_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "gathered_bytes_per_launch": gathered,
        },
    }
    # the page rebuilds the plan every 4 denoising steps and reuses it:
    # one selector + plan and four attention calls, per attention call
    def reuse4():
        bsa.bsa_select_scores(q, k, 128, kvb, C, c["kmeans_iters"], scores=scores, workspace=ws)
        bsa.bsa_sip_plan(scores, s, mode, seed=args.seed, idx=idx, bias=bias, count=cnt)
        for _ in range(4):
            bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, out=out)
    rec["ms_per_step_plan_every_4"] = round(_time(reuse4, 3) / 4, 4)
    # the same step captured once into a HIP graph and replayed, as a serving
    # loop would run it (outside the timed region; no launch from the host)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    rec["ms_per_step_graph"] = round(_time(graph.replay, max(3, args.steps)), 4)
    del graph
    # one cold call (outside the timed region): a 512 MB write evicts the
    # Infinity Cache first
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush.fill_(3)
    c0, c1 = ev(), ev()
    c0.record(stream)
    bsa.bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kvb, out=out)
    c1.record(stream)
    torch.cuda.synchronize()
    rec["attn_ms_cold"] = round(c0.elapsed_time(c1), 4)
    del flush
    # the matrix units' measured rate on the attention kernel's instruction
    # (outside the timed region)
    peak_meas, _ = mfma_peak(PEAK_PROBE_GRID, PEAK_PROBE_ITERS, operands=0)
    peak_low, _ = mfma_peak(PEAK_PROBE_GRID, PEAK_PROBE_ITERS, operands=1)
    rec["roofline"].update({
        "peak_measured": round(peak_meas, 2),
        "frac_measured": round(attn_tf / peak_meas, 4),
        "peak_measured_by": "bsa_mfma_peak_probe, random bf16 operands: v_mfma_f32_32x32x16_bf16 "
                            f"from registers, {PEAK_PROBE_GRID} workgroups of 4 waves x "
                            f"{PEAK_PROBE_ITERS} rounds of 8 chains, best of 3 (bench.py --mfma-peak)",
        "peak_measured_low_entropy": round(peak_low, 2),
    })
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calib_bytes"] = n
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(c, args.seed, min(args.cpu_sample_heads, H))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
