"""Pins of the conditioning oracle (timestep embedding, two-time blend,
AdaLN projection) against closed forms, identities, library routines and
hand-worked values (CPU only).

A wrong frequency exponent, swapped cos/sin halves, a dropped bias or SiLU,
a transposed weight, a misplaced gate or a wrong table reshape each fail at
least one of these.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import conditioning as oc
from joint_video_audio_amd import synth

TOL = 1e-12


def close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, float(np.abs(a - b).max())


# ---------------------------------------------------------------- sinusoid

def test_sinusoid_at_zero_is_ones_then_zeros():
    s = oc.sinusoid([0.0], 256)
    close(s[0, :128], np.ones(128))
    close(s[0, 128:], np.zeros(128))


def test_sinusoid_first_pair_is_cos_sin_of_t():
    # frequency 0 is 1, so the first pair is (cos t, sin t); values of
    # cos(1), sin(1), cos(0.5), sin(0.5) to 16 digits.
    s = oc.sinusoid([1.0, 0.5], 256)
    close(s[:, 0], [0.5403023058681398, 0.8775825618903728])
    close(s[:, 128], [0.8414709848078965, 0.479425538604203])


def test_sinusoid_decade_frequencies():
    # With period 10^4 over 128 frequencies, frequency 32 is 10^-1, 64 is
    # 10^-2 and 96 is 10^-3: at t = 1 the pair angles are those numbers.
    s = oc.sinusoid([1.0], 256)[0]
    ang = np.arctan2(s[128:], s[:128])
    close(ang[[0, 32, 64, 96]], [1.0, 0.1, 0.01, 0.001])
    # the angles fall geometrically
    ratio = ang[1:] / ang[:-1]
    close(ratio, np.full(127, ratio[0]))


def test_sinusoid_pythagoras_and_angle_addition():
    t1, t2 = 0.37, 0.21
    a = oc.sinusoid([t1], 256)[0]
    b = oc.sinusoid([t2], 256)[0]
    c = oc.sinusoid([t1 + t2], 256)[0]
    close(a[:128] ** 2 + a[128:] ** 2, np.ones(128))
    close(c[:128], a[:128] * b[:128] - a[128:] * b[128:])
    close(c[128:], a[128:] * b[:128] + a[:128] * b[128:])


# ---------------------------------------------------------------- MLP

def test_silu_values():
    close(oc.silu(np.array([0.0, 1.0, -1.0])), [0.0, 0.7310585786300049, -0.2689414213699951])


def test_time_mlp_hand_worked():
    # freq_dim 2 (one frequency, 1), hidden 1, embed 1, t = 0: s = (1, 0);
    # h = 2*1 + 3*0 - 1 = 1; SiLU(1) = 0.7310585786300049;
    # e = 4 * 0.7310585786300049 + 0.5 = 3.4242343145200196.
    s = oc.sinusoid([0.0], 2)
    e = oc.time_mlp(s, np.array([[2.0, 3.0]]), np.array([-1.0]), np.array([[4.0]]), np.array([0.5]))
    close(e, [[3.4242343145200196]])
    # at t = pi/2: s = (0, 1); h = 3 - 1 = 2; SiLU(2) = 1.7615941559557646;
    # e = 4 * 1.7615941559557646 + 0.5 = 7.5463766238230585.
    s = oc.sinusoid([math.pi / 2], 2)
    e = oc.time_mlp(s, np.array([[2.0, 3.0]]), np.array([-1.0]), np.array([[4.0]]), np.array([0.5]))
    close(e, [[7.5463766238230585]])


def test_time_mlp_matches_torch_layers():
    rng = np.random.default_rng(3)
    w1, b1 = rng.standard_normal((40, 16)), rng.standard_normal(40)
    w2, b2 = rng.standard_normal((24, 40)), rng.standard_normal(24)
    t = rng.random(5)
    s = oc.sinusoid(t, 16)
    ref = F.linear(F.silu(F.linear(torch.from_numpy(s), torch.from_numpy(w1), torch.from_numpy(b1))),
                   torch.from_numpy(w2), torch.from_numpy(b2)).numpy()
    close(oc.time_mlp(s, w1, b1, w2, b2), ref)


def test_time_mlp_zero_second_layer_gives_bias():
    rng = np.random.default_rng(4)
    s = oc.sinusoid(rng.random(3), 8)
    e = oc.time_mlp(s, rng.standard_normal((6, 8)), rng.standard_normal(6), np.zeros((4, 6)), np.arange(4.0))
    close(e, np.tile(np.arange(4.0), (3, 1)))


# ---------------------------------------------------------------- two-time blend

def _emb(rng, f, h, e):
    return dict(w1=rng.standard_normal((h, f)), b1=rng.standard_normal(h), w2=rng.standard_normal((e, h)),
                b2=rng.standard_normal(e))


def test_two_time_blend_endpoints_and_linearity():
    rng = np.random.default_rng(5)
    base, endp = _emb(rng, 8, 12, 6), _emb(rng, 8, 12, 6)
    t, r = rng.random(4), rng.random(4)
    e_t = oc.time_mlp(oc.sinusoid(t, 8), **base)
    e_r = oc.time_mlp(oc.sinusoid(r, 8), **endp)
    close(oc.time_embedding(t, 8, base), e_t)
    close(oc.time_embedding(t, 8, base, r, endp, 0.0), e_t)
    close(oc.time_embedding(t, 8, base, r, endp, 1.0), e_r)
    g = 0.3
    close(oc.time_embedding(t, 8, base, r, endp, g), e_t + g * (e_r - e_t))


def test_two_time_with_identical_embedders_and_r_equal_t_is_the_base_embedding():
    # Conditioning rows keep r = t: with an adapter that changes nothing the
    # blend returns the base embedding for any gate.
    rng = np.random.default_rng(6)
    base = _emb(rng, 8, 12, 6)
    t = rng.random(5)
    close(oc.time_embedding(t, 8, base, None, dict(base), 0.7), oc.time_embedding(t, 8, base))


# ---------------------------------------------------------------- AdaLN table

def test_table_layout_by_one_hot_rows():
    # W_k row (c D + d) = unit vector at input j(k, c, d): the table entry is
    # SiLU(e_v[j]) plus its bias; this fixes the tag axis, the six-vector
    # reshape and the per-entry bias.
    T, D, E, n = 3, 4, 7, 5
    rng = np.random.default_rng(7)
    e = rng.standard_normal((n, E))
    w = np.zeros((T, 6 * D, E))
    jsel = rng.integers(0, E, size=(T, 6, D))
    for k in range(T):
        for c in range(6):
            for d in range(D):
                w[k, c * D + d, jsel[k, c, d]] = 1.0
    b = rng.standard_normal((T, 6 * D))
    tab = oc.adaln_table(e, w, b, D)
    assert tab.shape == (T, n, 6, D)
    a = e / (1.0 + np.exp(-e))
    for k in range(T):
        for v in range(n):
            for c in range(6):
                for d in range(D):
                    assert abs(tab[k, v, c, d] - (a[v, jsel[k, c, d]] + b[k, c * D + d])) < 1e-12


def test_table_matches_torch_per_tag_and_tags_are_separate():
    T, D, E, n = 3, 8, 16, 6
    rng = np.random.default_rng(8)
    e = rng.standard_normal((n, E))
    w = rng.standard_normal((T, 6 * D, E))
    b = rng.standard_normal((T, 6 * D))
    tab = oc.adaln_table(e, w, b, D)
    for k in range(T):
        ref = F.linear(F.silu(torch.from_numpy(e)), torch.from_numpy(w[k]), torch.from_numpy(b[k])).numpy()
        close(tab[k].reshape(n, 6 * D), ref)
    w2 = w.copy()
    w2[1] += 1.0
    tab2 = oc.adaln_table(e, w2, b, D)
    close(tab2[0], tab[0])
    close(tab2[2], tab[2])
    assert np.abs(tab2[1] - tab[1]).max() > 1e-3
    # permuting the timestep values permutes the table's second axis
    p = rng.permutation(n)
    close(oc.adaln_table(e[p], w, b, D), tab[:, p])
    # no bias given = zero bias
    close(oc.adaln_table(e, w, None, D), oc.adaln_table(e, w, np.zeros_like(b), D))


def test_synthetic_two_time_grid_diagonal_is_r_equal_t():
    dims = synth.ModelDims(hidden=256, num_heads=2, ffn_dim=256, num_tvals=16, dtype="f32")
    c = synth.make_conditioning(dims, two_time=True, freq_dim=16, hidden_dim=32, embed_dim=32)
    v = np.arange(16)
    assert np.all(c.t[v[v % 5 == 0]] == c.r[v[v % 5 == 0]])
    assert len(set(zip(c.t.tolist(), c.r.tolist()))) == 16
