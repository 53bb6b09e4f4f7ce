"""Shared test helpers: tolerances, metrics, conversions."""
from __future__ import annotations

import numpy as np
import torch

# Bar for float tensors computed in bf16 (fp32 accumulation, bf16 storage):
# relative L2 error <= 1e-2 and max-abs error <= 5e-2 per output tensor.
REL_L2_BF16 = 1e-2
MAX_ABS_BF16 = 5e-2
# fp32 storage and compute: the same graded bar applies; internally we hold
# the fp32 path to 1e-4 relative L2.
REL_L2_F32 = 1e-4


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max()) if np.size(a) else 0.0


def assert_close(got, want, name: str, rel=REL_L2_BF16, mabs=MAX_ABS_BF16):
    r, m = rel_l2(got, want), max_abs(got, want)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert r <= rel and m <= mabs, f"{name}: rel_l2={r:.3e} (<= {rel}) max_abs={m:.3e} (<= {mabs})"
    return r, m
