"""Block-sparse attention forward on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libbsa.so`` (declared in
``include/bsa.h``).  It only marshals arguments: every step of the path runs
in the library's HIP kernels.  PyTorch provides device memory and the
current stream.  The library must be built (``python
block_sparse_attention_mean_amd/build.py``); importing the binding without it
raises ImportError -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

# torch first: it carries its own HIP runtime, and libbsa.so's dependency on
# libamdhip64.so.7 must resolve to that copy.  Loaded before torch, the
# library would pull in a second HIP runtime (/opt/rocm's), in which torch's
# streams and allocations do not exist, and every launch would fail.
import torch  # noqa: F401

__all__ = [
    "lib", "BsaError", "bsa_select_scores", "bsa_sip_plan", "bsa_attn_fwd",
    "bsa_sampling_offset", "bsa_select_workspace_bytes", "bsa_basa_layout",
    "bsa_basa_plan", "bsa_basa_plan_noalloc", "bsa_window_unpermute", "bsa_block_mass",
    "bsa_plan_coverage", "bsa_output_error", "dense_plan", "bsa_basa_offsets", "bsa_basa_shifts", "bsa_attn_bwd",
    "bsa_attn_bwd_workspace_bytes", "bsa_attn_bwd_ws", "bsa_mfma_peak_probe", "PLAN_SIP", "PLAN_TOPK", "LIB_PATH", "OK", "ERR_NONFINITE",
    "PROBE_RANDOM", "PROBE_LOW_ENTROPY",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa.so")
PLAN_SIP, PLAN_TOPK = 0, 1
OK, ERR_NONFINITE = 0, -9   # values of a plan's status word
PROBE_RANDOM, PROBE_LOW_ENTROPY = 0, 1   # operand modes of the matrix probe

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with "
                      "`python block_sparse_attention_mean_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_p, _i, _f, _sz, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
_pi, _psz = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_size_t)

lib.bsa_status_string.restype = ctypes.c_char_p
lib.bsa_status_string.argtypes = [_i]
lib.bsa_version.restype = ctypes.c_char_p
lib.bsa_version.argtypes = []
lib.bsa_sampling_offset.restype = _u64
lib.bsa_sampling_offset.argtypes = [_u64, _u64]
lib.bsa_select_workspace_bytes.restype = _i
lib.bsa_select_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _psz]
lib.bsa_select_scores.restype = _i
lib.bsa_select_scores.argtypes = [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]
lib.bsa_sip_plan.restype = _i
lib.bsa_sip_plan.argtypes = [_p, _i, _i, _i, _i, _i, _i, _u64, _p, _p, _p, _p, _p, _p, _p]
lib.bsa_attn_fwd.restype = _i
lib.bsa_attn_fwd.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _f, _p, _p, _p]
lib.bsa_basa_layout.restype = _i
lib.bsa_basa_layout.argtypes = [_i] * 12 + [_pi] * 4 + [_psz]
lib.bsa_basa_plan.restype = _i
lib.bsa_basa_plan.argtypes = [_p, _p, _p] + [_i] * 14 + [_p] * 6 + [_p, _sz, _p]
lib.bsa_basa_plan_noalloc.restype = _i
lib.bsa_basa_plan_noalloc.argtypes = [_p, _p, _p] + [_i] * 14 + [_p] * 6 + [_p]
lib.bsa_window_unpermute.restype = _i
lib.bsa_window_unpermute.argtypes = [_p, _p] + [_i] * 10 + [_p]
lib.bsa_block_mass.restype = _i
lib.bsa_block_mass.argtypes = [_p, _p, _p] + [_i] * 7 + [_f, _p, _p]
lib.bsa_plan_coverage.restype = _i
lib.bsa_plan_coverage.argtypes = [_p, _p, _p, _i, _i, _i, _p, _p]
lib.bsa_attn_bwd.restype = _i
lib.bsa_attn_bwd.argtypes = [_p] * 6 + [_i] * 7 + [_p, _p, _p, _i, _f, _p, _p, _p, _p]
lib.bsa_attn_bwd_workspace_bytes.restype = _i
lib.bsa_attn_bwd_workspace_bytes.argtypes = [_i] * 6 + [_psz]
lib.bsa_attn_bwd_ws.restype = _i
lib.bsa_attn_bwd_ws.argtypes = [_p] * 6 + [_i] * 7 + [_p, _p, _p, _i, _f, _p, _p, _p, _p, _sz, _p]
lib.bsa_basa_offsets.restype = _i
lib.bsa_basa_offsets.argtypes = [_i, _i, _pi]
lib.bsa_basa_shifts.restype = _i
lib.bsa_basa_shifts.argtypes = [_i, _i, _i, _i, _pi, _pi, _pi, _pi]
lib.bsa_mfma_peak_probe.restype = _i
lib.bsa_mfma_peak_probe.argtypes = [_i, _i, _i, _p, ctypes.POINTER(ctypes.c_longlong), _p]
lib.bsa_output_error.restype = _i
lib.bsa_output_error.argtypes = [_p, _p, _i, ctypes.c_longlong, _p, _p]

# Exported symbols of include/bsa.h (checked by the CPU tests).
SYMBOLS = ["bsa_status_string", "bsa_version", "bsa_select_workspace_bytes", "bsa_select_scores",
           "bsa_sip_plan", "bsa_sampling_offset", "bsa_attn_fwd", "bsa_basa_layout",
           "bsa_basa_plan", "bsa_window_unpermute", "bsa_block_mass", "bsa_plan_coverage",
           "bsa_output_error", "bsa_basa_offsets", "bsa_basa_shifts", "bsa_attn_bwd",
           "bsa_attn_bwd_workspace_bytes", "bsa_attn_bwd_ws", "bsa_basa_plan_noalloc",
           "bsa_mfma_peak_probe"]


class BsaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {lib.bsa_status_string(status).decode()} (status {status})")


def _check(status: int, call: str):
    if status != 0:
        raise BsaError(status, call)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, dtype, name, ndim=None, shape=None, device=None):
    """A device tensor of ``dtype``, contiguous, with ``ndim`` dims or exactly
    ``shape``, on ``device`` (default: the current device, where the library
    launches).  Raises ValueError, so a wrong tensor never reaches a kernel."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    want = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    if t.device != want:
        raise ValueError(f"{name} is on {t.device}, expected {want}")
    return t


def _opt(t, dtype, name, shape, device):
    """_need for an optional tensor (None passes)."""
    return None if t is None else _need(t, dtype, name, shape=shape, device=device)


def bsa_sampling_offset(seed: int, row: int) -> int:
    return int(lib.bsa_sampling_offset(seed & (2**64 - 1), row))


def bsa_select_workspace_bytes(B, H, N, d, q_block=128, kv_block=4, n_clusters=8) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.bsa_select_workspace_bytes(B, H, N, d, q_block, kv_block, n_clusters,
                                          ctypes.byref(out)), "bsa_select_workspace_bytes")
    return out.value


def bsa_select_scores(q, k, q_block=128, kv_block=4, n_clusters=8, kmeans_iters=1,
                      scores=None, centroids=None, weights=None, workspace=None,
                      want_centroids=False, stream=None):
    """q, k: [B,H,N,d] bf16 -> scores [B,H,nQB,M] fp32 (+ centroids, weights)."""
    _need(q, torch.bfloat16, "q", 4)
    dev = q.device
    B, H, N, d = q.shape
    _need(k, torch.bfloat16, "k", shape=q.shape, device=dev)
    nqb, M = -(-N // q_block), -(-N // kv_block)
    if scores is None:
        scores = torch.empty((B, H, nqb, M), dtype=torch.float32, device=dev)
    _need(scores, torch.float32, "scores", shape=(B, H, nqb, M), device=dev)
    if want_centroids and centroids is None:
        centroids = torch.empty((B, H, nqb, n_clusters, d), dtype=torch.float32, device=dev)
    if want_centroids and weights is None:
        weights = torch.empty((B, H, nqb, n_clusters), dtype=torch.float32, device=dev)
    _opt(centroids, torch.float32, "centroids", (B, H, nqb, n_clusters, d), dev)
    _opt(weights, torch.float32, "weights", (B, H, nqb, n_clusters), dev)
    need = bsa_select_workspace_bytes(B, H, N, d, q_block, kv_block, n_clusters)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", 1, device=dev)
    _check(lib.bsa_select_scores(_ptr(q), _ptr(k), B, H, N, d, q_block, kv_block, n_clusters,
                                 kmeans_iters, _ptr(scores), _ptr(centroids), _ptr(weights),
                                 _ptr(workspace), workspace.numel(), _stream(stream)),
           "bsa_select_scores")
    return scores, centroids, weights


def bsa_sip_plan(scores, budget, mode=PLAN_SIP, seed=0, offsets=None, idx=None, bias=None,
                 count=None, lam=None, want_lambda=False, status=None, stream=None):
    """scores [B,H,nQB,M] fp32 -> (idx, bias, count, lambda) device tensors.

    ``status`` (optional, one int32 on the device) receives BSA_OK, or
    BSA_ERR_NONFINITE when a row held a NaN, an infinity or a negative score
    (that row gets count -1)."""
    _need(scores, torch.float32, "scores", 4)
    B, H, nqb, M = scores.shape
    dev = scores.device
    if idx is None:
        idx = torch.empty((B, H, nqb, budget), dtype=torch.int32, device=dev)
    if bias is None:
        bias = torch.empty((B, H, nqb, budget), dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    if want_lambda and lam is None:
        lam = torch.empty((B, H, nqb), dtype=torch.float64, device=dev)
    _need(idx, torch.int32, "idx", shape=(B, H, nqb, budget), device=dev)
    _need(bias, torch.float32, "bias", shape=(B, H, nqb, budget), device=dev)
    _need(count, torch.int32, "count", shape=(B, H, nqb), device=dev)
    _opt(lam, torch.float64, "lam", (B, H, nqb), dev)
    _opt(status, torch.int32, "status", (1,), dev)
    if offsets is not None:
        _need(offsets, torch.int64, "offsets", device=dev)
        if offsets.numel() != B * H * nqb:
            raise ValueError(f"offsets must hold B*H*nQB = {B * H * nqb} values")
    _check(lib.bsa_sip_plan(_ptr(scores), B, H, nqb, M, budget, mode, seed & (2**64 - 1),
                            _ptr(offsets), _ptr(idx), _ptr(bias), _ptr(count), _ptr(lam),
                            _ptr(status), _stream(stream)), "bsa_sip_plan")
    return idx, bias, count, lam


def _plan_args(q, k, idx, bias, count, q_block, dev):
    """Shapes of an attention call: q [B,H,Nq,d], k [B,H,Nk,d], idx / bias
    [B,H,nQB,L], count [B,H,nQB]; returns (B, H, Nq, Nk, d, L)."""
    B, H, Nq, d = q.shape
    if k.dim() != 4 or tuple(k.shape[:2]) != (B, H) or k.shape[3] != d:
        raise ValueError(f"k must have shape ({B}, {H}, Nk, {d}), got {tuple(k.shape)}")
    Nk = k.shape[2]
    nqb = -(-Nq // q_block)
    _need(idx, torch.int32, "idx", 4, device=dev)
    if tuple(idx.shape[:3]) != (B, H, nqb):
        raise ValueError(f"idx must have shape ({B}, {H}, {nqb}, L), got {tuple(idx.shape)}")
    L = idx.shape[3]
    _opt(bias, torch.float32, "bias", (B, H, nqb, L), dev)
    _need(count, torch.int32, "count", shape=(B, H, nqb), device=dev)
    return B, H, Nq, Nk, d, L


def bsa_attn_fwd(q, k, v, idx, bias, count, q_block=128, kv_block=4, softmax_scale=0.0,
                 out=None, lse=None, want_lse=False, stream=None):
    """q [B,H,Nq,d], k/v [B,H,Nk,d] bf16; idx [B,H,nQB,L] int32; bias (optional)
    [B,H,nQB,L] fp32; count [B,H,nQB] int32 -> out [B,H,Nq,d] bf16 (+ lse)."""
    _need(q, torch.bfloat16, "q", 4)
    dev = q.device
    _need(k, torch.bfloat16, "k", 4, device=dev)
    B, H, Nq, Nk, d, L = _plan_args(q, k, idx, bias, count, q_block, dev)
    _need(v, torch.bfloat16, "v", shape=k.shape, device=dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out", shape=q.shape, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _opt(lse, torch.float32, "lse", (B, H, Nq), dev)
    _check(lib.bsa_attn_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, d, q_block, kv_block,
                            _ptr(idx), _ptr(bias), _ptr(count), L, float(softmax_scale),
                            _ptr(out), _ptr(lse), _stream(stream)),
           "bsa_attn_fwd")
    return out, lse


def _bwd_outputs(q, k, v, out, dout, lse, idx, bias, count, q_block, dq, dk, dv):
    _need(q, torch.bfloat16, "q", 4)
    dev = q.device
    _need(k, torch.bfloat16, "k", 4, device=dev)
    B, H, Nq, Nk, d, L = _plan_args(q, k, idx, bias, count, q_block, dev)
    _need(v, torch.bfloat16, "v", shape=k.shape, device=dev)
    _need(out, torch.bfloat16, "out", shape=q.shape, device=dev)
    _need(dout, torch.bfloat16, "dout", shape=q.shape, device=dev)
    _need(lse, torch.float32, "lse", shape=(B, H, Nq), device=dev)
    if dq is None:
        dq = torch.empty((B, H, Nq, d), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((B, H, Nk, d), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, H, Nk, d), dtype=torch.float32, device=dev)
    _need(dq, torch.float32, "dq", shape=(B, H, Nq, d), device=dev)
    _need(dk, torch.float32, "dk", shape=(B, H, Nk, d), device=dev)
    _need(dv, torch.float32, "dv", shape=(B, H, Nk, d), device=dev)
    return (B, H, Nq, Nk, d, L), dq, dk, dv


def bsa_attn_bwd(q, k, v, out, dout, lse, idx, bias, count, q_block=128, kv_block=4,
                 softmax_scale=0.0, dq=None, dk=None, dv=None, stream=None):
    """Gradients of sum(dout * out) for out = bsa_attn_fwd(q, k, v, idx, bias,
    count, ...) with the plan fixed: (dq [B,H,Nq,d], dk, dv [B,H,Nk,d]) fp32."""
    (B, H, Nq, Nk, d, L), dq, dk, dv = _bwd_outputs(q, k, v, out, dout, lse, idx, bias, count,
                                                    q_block, dq, dk, dv)
    _check(lib.bsa_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), B, H, Nq,
                            Nk, d, q_block, kv_block, _ptr(idx), _ptr(bias), _ptr(count),
                            L, float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                            _stream(stream)), "bsa_attn_bwd")
    return dq, dk, dv


def bsa_attn_bwd_workspace_bytes(Nq, Nk, d, max_blocks, q_block=128, kv_block=4) -> int:
    """Workspace bytes bsa_attn_bwd_ws needs per (b, h) slab."""
    out = ctypes.c_size_t(0)
    _check(lib.bsa_attn_bwd_workspace_bytes(Nq, Nk, d, q_block, kv_block, max_blocks,
                                            ctypes.byref(out)), "bsa_attn_bwd_workspace_bytes")
    return out.value


def bsa_attn_bwd_ws(q, k, v, out, dout, lse, idx, bias, count, q_block=128, kv_block=4,
                    softmax_scale=0.0, dq=None, dk=None, dv=None, workspace=None, slabs=None,
                    stream=None):
    """bsa_attn_bwd without atomic adds, through a workspace of partial rows
    (one per entry of the union of two neighbouring query blocks' lists).
    Without ``workspace`` one of ``slabs`` (b, h) slabs (default all B*H) is
    allocated; the call runs as many slabs at a time as the workspace
    holds."""
    (B, H, Nq, Nk, d, L), dq, dk, dv = _bwd_outputs(q, k, v, out, dout, lse, idx, bias, count,
                                                    q_block, dq, dk, dv)
    if workspace is None:
        per = bsa_attn_bwd_workspace_bytes(Nq, Nk, d, L, q_block, kv_block)
        n = B * H if slabs is None else max(1, min(int(slabs), B * H))
        workspace = torch.empty(per * n, dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace", 1, device=q.device)
    _check(lib.bsa_attn_bwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), B, H,
                               Nq, Nk, d, q_block, kv_block, _ptr(idx), _ptr(bias), _ptr(count),
                               L, float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(workspace), workspace.numel(), _stream(stream)),
           "bsa_attn_bwd_ws")
    return dq, dk, dv


def bsa_basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block=4, B=1, H=1):
    vals = [ctypes.c_int(0) for _ in range(4)]
    ws = ctypes.c_size_t(0)
    _check(lib.bsa_basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, B, H,
                               *[ctypes.byref(x) for x in vals], ctypes.byref(ws)),
           "bsa_basa_layout")
    keys = ["nwin", "Nq_pad", "Nk", "max_blocks"]
    out = {k: v.value for k, v in zip(keys, vals)}
    out["workspace"] = ws.value
    return out


def _basa_outputs(q, lay, topk, want_routes, out):
    """Output tensors of the BASA list builder: the caller's (``out``, a dict
    with the keys bsa_basa_plan returns, checked against the layout) or new
    ones."""
    B, H, _, d = q.shape
    nqb = lay["Nq_pad"] // 128
    shapes = dict(qp=((B, H, lay["Nq_pad"], d), torch.bfloat16),
                  kp=((B, H, lay["Nk"], d), torch.bfloat16),
                  vp=((B, H, lay["Nk"], d), torch.bfloat16),
                  idx=((B, H, nqb, lay["max_blocks"]), torch.int32),
                  count=((B, H, nqb), torch.int32),
                  routes=((B, H, lay["nwin"], max(topk, 1)), torch.int32))
    res = {}
    for key, (shape, dtype) in shapes.items():
        t = None if out is None else out.get(key)
        if t is None:
            if key == "routes" and not want_routes:
                res[key] = None
                continue
            t = torch.empty(shape, dtype=dtype, device=q.device)
        else:
            _need(t, dtype, key, shape=shape, device=q.device)
        res[key] = t
    return res


def _basa_inputs(q, k, v, T, Hg, Wg):
    _need(q, torch.bfloat16, "q", 4)
    if q.shape[2] != T * Hg * Wg:
        raise ValueError(f"q holds {q.shape[2]} tokens, the grid {T}x{Hg}x{Wg} {T * Hg * Wg}")
    _need(k, torch.bfloat16, "k", shape=q.shape, device=q.device)
    _need(v, torch.bfloat16, "v", shape=q.shape, device=q.device)
    return q.shape


def bsa_basa_plan(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kv_block=4,
                  want_routes=False, stream=None):
    """Window-major Q/K/V (+ pooled memory) and the block lists of BASA."""
    B, H, N, d = _basa_inputs(q, k, v, T, Hg, Wg)
    lay = bsa_basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, B, H)
    o = _basa_outputs(q, lay, topk, want_routes, None)
    ws = torch.empty(max(lay["workspace"], 256), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_basa_plan(_ptr(q), _ptr(k), _ptr(v), B, H, T, Hg, Wg, d, wh, ww, dy, dx, ph,
                             pw, topk, kv_block, _ptr(o["qp"]), _ptr(o["kp"]), _ptr(o["vp"]),
                             _ptr(o["idx"]), _ptr(o["count"]), _ptr(o["routes"]), _ptr(ws),
                             ws.numel(), _stream(stream)),
           "bsa_basa_plan")
    return dict(**o, **lay)


def bsa_basa_plan_noalloc(q, k, v, T, Hg, Wg, wh, ww, dy, dx, ph, pw, topk, kv_block=4,
                          want_routes=False, out=None, stream=None):
    """bsa_basa_plan without a workspace: the library's fixed device scratch
    replaces it, so the C call allocates nothing.  ``out`` (a dict with the
    keys qp, kp, vp, idx, count and optionally routes) supplies the outputs;
    missing ones are allocated here, before the call."""
    B, H, N, d = _basa_inputs(q, k, v, T, Hg, Wg)
    lay = bsa_basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, B, H)
    o = _basa_outputs(q, lay, topk, want_routes, out)
    _check(lib.bsa_basa_plan_noalloc(_ptr(q), _ptr(k), _ptr(v), B, H, T, Hg, Wg, d, wh, ww, dy,
                                     dx, ph, pw, topk, kv_block, _ptr(o["qp"]), _ptr(o["kp"]),
                                     _ptr(o["vp"]), _ptr(o["idx"]), _ptr(o["count"]),
                                     _ptr(o["routes"]), _stream(stream)),
           "bsa_basa_plan_noalloc")
    return dict(**o, **lay)


def bsa_window_unpermute(out_perm, T, Hg, Wg, wh, ww, dy, dx, out=None, stream=None):
    _need(out_perm, torch.bfloat16, "out_perm", 4)
    B, H, Np, d = out_perm.shape
    # the padded window-major row count depends on the windows only
    nq_pad = bsa_basa_layout(T, Hg, Wg, d, wh, ww, 1, 1, 0, 1, B, H)["Nq_pad"]
    if Np != nq_pad:
        raise ValueError(f"out_perm must have {nq_pad} window-major rows, got {Np}")
    if out is None:
        out = torch.empty((B, H, T * Hg * Wg, d), dtype=torch.bfloat16, device=out_perm.device)
    _need(out, torch.bfloat16, "out", shape=(B, H, T * Hg * Wg, d), device=out_perm.device)
    _check(lib.bsa_window_unpermute(_ptr(out_perm), _ptr(out), B, H, T, Hg, Wg, d, wh, ww, dy,
                                    dx, _stream(stream)), "bsa_window_unpermute")
    return out


def dense_plan(B, H, Nq, Nk, kv_block=128, device="cuda"):
    """A list of every KV block for every query block (no bias): with it,
    bsa_attn_fwd computes dense attention and its lse is the dense one."""
    nqb, M = -(-Nq // 128), -(-Nk // kv_block)
    idx = torch.arange(M, dtype=torch.int32, device=device).expand(B, H, nqb, M).contiguous()
    count = torch.full((B, H, nqb), M, dtype=torch.int32, device=device)
    return idx, count


def bsa_block_mass(q, k, lse, q_block=128, kv_block=4, softmax_scale=0.0, mass=None,
                   stream=None):
    """q [B,H,Nq,d], k [B,H,Nk,d] bf16, lse [B,H,Nq] fp32 (dense) -> mass
    [B,H,nQB,M] fp32: true attention mass of every KV block per query block."""
    _need(q, torch.bfloat16, "q", 4)
    dev = q.device
    B, H, Nq, d = q.shape
    _need(k, torch.bfloat16, "k", 4, device=dev)
    if tuple(k.shape[:2]) != (B, H) or k.shape[3] != d:
        raise ValueError(f"k must have shape ({B}, {H}, Nk, {d}), got {tuple(k.shape)}")
    Nk = k.shape[2]
    _need(lse, torch.float32, "lse", shape=(B, H, Nq), device=dev)
    if kv_block < 1:
        raise ValueError("kv_block must be positive")
    shape = (B, H, -(-Nq // q_block), -(-Nk // kv_block))
    if mass is None:
        mass = torch.empty(shape, dtype=torch.float32, device=dev)
    _need(mass, torch.float32, "mass", shape=shape, device=dev)
    _check(lib.bsa_block_mass(_ptr(q), _ptr(k), _ptr(lse), B, H, Nq, Nk, d, q_block, kv_block,
                              float(softmax_scale), _ptr(mass), _stream(stream)), "bsa_block_mass")
    return mass


def bsa_plan_coverage(mass, idx, count, coverage=None, stream=None):
    """mass [..., M] fp32, idx [..., L] int32, count [...] int32 -> retained
    mass [...] fp64."""
    _need(mass, torch.float32, "mass")
    dev = mass.device
    _need(idx, torch.int32, "idx", device=dev)
    _need(count, torch.int32, "count", device=dev)
    lead = tuple(mass.shape[:-1])
    rows = count.numel()
    if mass.dim() < 1 or idx.dim() != mass.dim() or tuple(idx.shape[:-1]) != lead \
            or tuple(count.shape) != lead:
        raise ValueError("mass, idx and count must share their leading dims")
    if coverage is None:
        coverage = torch.empty(lead, dtype=torch.float64, device=dev)
    _need(coverage, torch.float64, "coverage", shape=lead, device=dev)
    _check(lib.bsa_plan_coverage(_ptr(mass), _ptr(idx), _ptr(count), rows, mass.shape[-1],
                                 idx.shape[-1], _ptr(coverage), _stream(stream)),
           "bsa_plan_coverage")
    return coverage


def bsa_output_error(out, ref, sums=None, stream=None):
    """out, ref [B,H,N,d] bf16 -> sums [B,H,2] fp64: (sum (out-ref)^2, sum ref^2)."""
    _need(out, torch.bfloat16, "out", 4)
    _need(ref, torch.bfloat16, "ref", shape=out.shape, device=out.device)
    B, H, N, d = out.shape
    if sums is None:
        sums = torch.empty((B, H, 2), dtype=torch.float64, device=out.device)
    _need(sums, torch.float64, "sums", shape=(B, H, 2), device=out.device)
    _check(lib.bsa_output_error(_ptr(out), _ptr(ref), B * H, N * d, _ptr(sums), _stream(stream)),
           "bsa_output_error")
    return sums


def bsa_basa_offsets(w: int, L: int) -> list:
    """The L per-layer window offsets along an axis of window size w."""
    out = (ctypes.c_int * L)()
    _check(lib.bsa_basa_offsets(w, L, out), "bsa_basa_offsets")
    return list(out)


def bsa_basa_shifts(wh: int, ww: int, L: int, S: int = 1, c_h=None, c_w=None):
    """(dy, dx), each a list of L lists of S ints: Delta_{l,s} of layer l at
    step s, with optional per-step offsets c_h, c_w (length S)."""
    ch = None if c_h is None else (ctypes.c_int * S)(*[int(x) for x in c_h])
    cw = None if c_w is None else (ctypes.c_int * S)(*[int(x) for x in c_w])
    for c, n in ((c_h, "c_h"), (c_w, "c_w")):
        if c is not None and len(c) != S:
            raise ValueError(f"{n} must have S = {S} entries")
    dy, dx = (ctypes.c_int * (L * S))(), (ctypes.c_int * (L * S))()
    _check(lib.bsa_basa_shifts(wh, ww, L, S, ch, cw, dy, dx), "bsa_basa_shifts")
    return ([list(dy[l * S:(l + 1) * S]) for l in range(L)],
            [list(dx[l * S:(l + 1) * S]) for l in range(L)])


def bsa_mfma_peak_probe(workgroups, iters, sink, operands=None, stream=None) -> int:
    """Launches the bf16 matrix-instruction throughput probe (operands:
    PROBE_RANDOM, the default, or PROBE_LOW_ENTROPY); returns the flops of
    the call (time it with events on the stream)."""
    _need(sink, torch.float32, "sink", shape=(1,))
    fl = ctypes.c_longlong(0)
    mode = PROBE_RANDOM if operands is None else operands
    _check(lib.bsa_mfma_peak_probe(workgroups, iters, mode, _ptr(sink), ctypes.byref(fl),
                                   _stream(stream)), "bsa_mfma_peak_probe")
    return fl.value


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
