"""Shared test helpers: tolerances, metrics, conversions."""
from __future__ import annotations

import numpy as np
import torch

# Bar for float tensors computed in bf16 (fp32 accumulation, bf16 storage):
# relative L2 error <= 1e-2 and max-abs error <= 5e-2 per output tensor.
REL_L2_BF16 = 1e-2
MAX_ABS_BF16 = 5e-2
# fp32 storage and compute: the same graded bar applies; internally we hold
# the fp32 path to 1e-4 relative L2 and 1e-3 max-abs (fp32 rounding of sums
# over at most a few thousand terms of size ~1 stays near 1e-5).
REL_L2_F32 = 1e-4
MAX_ABS_F32 = 1e-3


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


def half_ulp_bf16(want) -> np.ndarray:
    """Half the bf16 spacing at |want| (8 significant bits): the largest
    distance between a value and its round-to-nearest bf16 neighbour."""
    a = np.abs(np.asarray(want, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def assert_close_bf16_storage(got, want, name: str, rel=REL_L2_BF16, mabs=MAX_ABS_BF16):
    """The bar for a tensor STORED in bf16: relative L2 <= rel and, per
    element, |got - want| <= mabs + half a bf16 ulp of want. For |want| >= 16
    half an ulp is 0.0625 > 5e-2, so even the exactly rounded value would
    miss a plain max-abs of 5e-2; the allowance is that storage rounding and
    nothing more. Returns (rel_l2, max_abs, worst excess over mabs)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r, m = rel_l2(got, want), max_abs(got, want)
    excess = float((np.abs(got - want) - half_ulp_bf16(want)).max()) if got.size else 0.0
    assert r <= rel and excess <= mabs, \
        f"{name}: rel_l2={r:.3e} (<= {rel}) max_abs={m:.3e}, beyond half a bf16 ulp {excess:.3e} (<= {mabs})"
    return r, m, excess
