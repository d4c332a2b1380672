"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

# Parity tolerances on bf16 attention outputs (max-abs, mean-abs).
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3
# Relative tolerance on fp32 block scores.
SCORE_REL = 1e-4


def say(*msg):
    """Print-and-flush so a failing GPU step names its case."""
    print(*msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> fp64 numpy (exact)."""
    u = t.detach().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def assert_attn_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    diff = np.abs(got - want)
    mx, mean = float(diff.max()), float(diff.mean())
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= ATTN_MAX_ABS, f"{what}: max-abs {mx}"
    assert mean <= ATTN_MEAN_ABS, f"{what}: mean-abs {mean}"
