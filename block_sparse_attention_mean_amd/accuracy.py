"""Accuracy diagnostics of sampling plans on given activations.

Measures, with the library's kernels only, the quantities behind the
AB-Attention page's accuracy claims (onedev.kr/papers/1521):

* retained mass of an oracle top-k against KV block size (section
  "무엇과 다른가": the pages report it rising as the blocks shrink from
  128 to 4 tokens);
* output error against dense attention of SIP and of an oracle top-k at the
  same block size (section "어떻게 쓰나");
* the ablation variants of section "전제와 한계" (fixed sparsity): segment
  means instead of k-means, top-k on the selector's scores instead of SIP,
  SIP's sample without its 1/pi weighting, uniform sampling (no scores),
  selection at the 128-token execution tile (``ibcs_sip_kv128``), and the
  block-size sweep (``ibcs_sip_kv<b>``).

Every budget is a token budget, the same for every block size: a plan at
kv_block b lists round(tokens / b) blocks.  Dense attention is
bsa_attn_fwd over every block (128-token blocks, no bias); its LSE is the
normaliser of bsa_block_mass.  Errors are relative Frobenius errors per
head; retained masses are query-weighted means over the query blocks.
"""
from __future__ import annotations

import numpy as np

from . import (PLAN_SIP, PLAN_TOPK, bsa_attn_fwd, bsa_block_mass, bsa_output_error,
               bsa_plan_coverage, bsa_select_scores, bsa_sip_plan, dense_plan)

KV_SWEEP = (128, 64, 32, 16, 8, 4)


def dense_reference(q, k, v):
    """Dense attention output and its natural-log LSE."""
    B, H, Nq, _ = q.shape
    idx, cnt = dense_plan(B, H, Nq, k.shape[2], 128, device=q.device)
    return bsa_attn_fwd(q, k, v, idx, None, cnt, 128, 128, want_lse=True)


def _blocks(tokens: int, kv_block: int, M: int) -> int:
    return max(1, min(M, int(round(tokens / kv_block))))


def _query_weights(Nq: int) -> np.ndarray:
    n = np.full(-(-Nq // 128), 128.0)
    n[-1] = Nq - 128 * (len(n) - 1)
    return n / Nq


def relative_errors(out, ref) -> np.ndarray:
    """[B, H] relative Frobenius errors of out against ref."""
    s = bsa_output_error(out, ref).cpu().numpy()
    return np.sqrt(s[..., 0] / s[..., 1])


def retained_mass(mass, idx, count, Nq: int) -> np.ndarray:
    """[B, H] query-weighted mean of the mass a plan keeps."""
    cov = bsa_plan_coverage(mass, idx, count).cpu().numpy()
    return (cov * _query_weights(Nq)).sum(axis=-1)


def oracle_topk_curve(q, k, lse, tokens: int, kv_blocks=KV_SWEEP) -> dict:
    """{kv_block: [B, H] retained mass of the oracle top-k at that size}."""
    Nq = q.shape[2]
    out = {}
    for b in kv_blocks:
        mass = bsa_block_mass(q, k, lse, 128, b)
        s = _blocks(tokens, b, mass.shape[-1])
        idx, _, cnt, _ = bsa_sip_plan(mass, s, PLAN_TOPK)
        out[b] = retained_mass(mass, idx, cnt, Nq)
        del mass
    return out


def _run(q, k, v, ref, idx, bias, cnt, kv_block, mass=None):
    o, _ = bsa_attn_fwd(q, k, v, idx, bias, cnt, 128, kv_block)
    r = {"error": relative_errors(o, ref)}
    if mass is not None:
        r["retained_mass"] = retained_mass(mass, idx, cnt, q.shape[2])
    return r


def variants(q, k, v, ref, lse, tokens: int, seed: int = 0, n_clusters: int = 8,
             kmeans_iters: int = 1, kv_sweep=KV_SWEEP) -> dict:
    """{name: {"error": [B,H], "retained_mass": [B,H] (4-token variants)}}."""
    import torch
    Nq = q.shape[2]
    res = {}
    mass4 = bsa_block_mass(q, k, lse, 128, 4)
    M4 = mass4.shape[-1]
    s4 = _blocks(tokens, 4, M4)

    S, _, _ = bsa_select_scores(q, k, 128, 4, n_clusters, kmeans_iters)
    idx, bias, cnt, _ = bsa_sip_plan(S, s4, PLAN_SIP, seed=seed)
    res["ibcs_sip"] = _run(q, k, v, ref, idx, bias, cnt, 4, mass4)
    res["ibcs_sip_no_weighting"] = _run(q, k, v, ref, idx, None, cnt, 4, mass4)
    ti, _, tc, _ = bsa_sip_plan(S, s4, PLAN_TOPK)
    res["ibcs_topk"] = _run(q, k, v, ref, ti, None, tc, 4, mass4)
    del S

    S0, _, _ = bsa_select_scores(q, k, 128, 4, n_clusters, 0)
    i0, b0, c0, _ = bsa_sip_plan(S0, s4, PLAN_SIP, seed=seed)
    res["segment_means_sip"] = _run(q, k, v, ref, i0, b0, c0, 4, mass4)
    del S0

    U = torch.ones((q.shape[0], q.shape[1], -(-Nq // 128), M4), dtype=torch.float32,
                   device=q.device)
    iu, bu, cu, _ = bsa_sip_plan(U, s4, PLAN_SIP, seed=seed)
    res["uniform_sampling"] = _run(q, k, v, ref, iu, bu, cu, 4, mass4)
    del U

    oi, _, oc, _ = bsa_sip_plan(mass4, s4, PLAN_TOPK)
    res["oracle_topk"] = _run(q, k, v, ref, oi, None, oc, 4, mass4)
    si, sb, sc, _ = bsa_sip_plan(mass4, s4, PLAN_SIP, seed=seed)
    res["oracle_sip"] = _run(q, k, v, ref, si, sb, sc, 4, mass4)
    del mass4

    for b in kv_sweep:
        Sb, _, _ = bsa_select_scores(q, k, 128, b, n_clusters, kmeans_iters)
        sb_ = _blocks(tokens, b, Sb.shape[-1])
        ib, bb, cb, _ = bsa_sip_plan(Sb, sb_, PLAN_SIP, seed=seed)
        res[f"ibcs_sip_kv{b}"] = _run(q, k, v, ref, ib, bb, cb, b)
        del Sb
    return res
