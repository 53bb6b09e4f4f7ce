"""Pins of the denoising-step oracle (unmerged LoRA, timestep shift, Euler
update) against merged weights, closed forms and hand-worked values (CPU
only)."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import step as os_


def close(a, b, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.abs(a - b).max() <= tol * max(1.0, float(np.abs(b).max())), float(np.abs(a - b).max())


def test_unmerged_lora_equals_the_merged_weight():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 40))
    w = rng.standard_normal((24, 40))
    a = rng.standard_normal((8, 40))
    b = rng.standard_normal((24, 8))
    for scale in (1.0, 0.5, 0.0):
        got = os_.lora_linear(x, w, a, b, alpha=16.0, rank=8, scale=scale)
        merged = os_.lora_merged_weight(w, a, b, 16.0, 8, scale)
        close(got, F.linear(torch.from_numpy(x), torch.from_numpy(merged)).numpy(), 1e-10)
    # scale 0, or a zero B (how a fresh PEFT adapter starts), leave the base layer
    close(os_.lora_linear(x, w, a, b, 16.0, 8, 0.0), x @ w.T)
    close(os_.lora_linear(x, w, a, np.zeros_like(b), 16.0, 8, 1.0), x @ w.T)


def test_lora_rank_one_hand_worked():
    # x = (1, 2), W = 0, A = (3, 4) (rank 1), B = (5,), alpha = rank = 1:
    # x A^T = 11, times B = 55
    got = os_.lora_linear([[1.0, 2.0]], [[0.0, 0.0]], [[3.0, 4.0]], [[5.0]], alpha=1.0, rank=1)
    close(got, [[55.0]])
    # alpha / rank = 2 doubles it
    close(os_.lora_linear([[1.0, 2.0]], [[0.0, 0.0]], [[3.0, 4.0]], [[5.0]], alpha=2.0, rank=1), [[110.0]])


def test_shift_closed_forms():
    s = np.array([0.0, 0.25, 0.5, 1.0])
    # fixed points 0 and 1; shift 1 is the identity; shift 3 at 1/2 gives 3/4;
    # shift 12 at 1/4 gives 3 / (1 + 11/4) = 0.8
    close(os_.shift_sigmas(s, 1.0), s)
    close(os_.shift_sigmas(s, 3.0)[[0, 2, 3]], [0.0, 0.75, 1.0])
    close(os_.shift_sigmas(s, 12.0)[1], 0.8)
    # monotone: larger shifts keep more noise
    assert np.all(os_.shift_sigmas(s[1:3], 12.0) > os_.shift_sigmas(s[1:3], 3.0))


def test_euler_step_moves_along_the_velocity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 6))
    v = rng.standard_normal((5, 6))
    now = np.array([1.0, 0.75, 0.5, 0.5, 0.25])
    nxt = np.array([0.75, 0.5, 0.5, 0.0, 0.0])
    y = os_.euler_step(x, v, now, nxt)
    close(y[2], x[2])                    # equal sigmas: the row stays
    close(y[3], x[3] - 0.5 * v[3])
    # with v = x1 - x0 (the straight flow between noise x1 and data x0) a
    # step from sigma to 0 lands on x0
    x0, x1 = rng.standard_normal(6), rng.standard_normal(6)
    xs = 0.75 * x1 + 0.25 * x0
    close(os_.euler_step(xs[None], (x1 - x0)[None], [0.75], [0.0])[0], x0)
