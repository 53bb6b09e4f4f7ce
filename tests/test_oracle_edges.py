"""Pins of the model-edge oracle (input projections with the scatter into
the packed sequence, norm_out, output heads with the gather) against
library routines, closed forms, hand-worked values and index bookkeeping
(CPU only).

A row sent to the wrong packed position, a transposed weight, a dropped bias,
norm_out without its weight or bias, or outputs in the wrong row order each
fail at least one of these.
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import edges as oe
from joint_video_audio_amd import synth

TOL = 1e-12


def close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, float(np.abs(a - b).max())


def small_layout(pads=5, seed=0):
    dims = synth.ModelDims(hidden=32, num_heads=2, ffn_dim=64, num_tvals=4, dtype="f32")
    segs = [("text", 7), ("cond", 6, (1, 2, 3)), ("audio", 5), ("video", 24, (2, 3, 4))]
    wl = synth.make_custom(dims, segs, (2, 3, 4), pads, seed=seed)
    return dims, wl.layout


def test_one_hot_projections_place_rows_exactly():
    dims, L = small_layout()
    rng = np.random.default_rng(1)
    B, D, Cv, Ca = 2, dims.hidden, 6, 4
    nv, na, nt = len(L.video_indices), len(L.audio_indices), len(L.text_indices)
    video = rng.standard_normal((B, nv, Cv))
    audio = rng.standard_normal((B, na, Ca))
    text = rng.standard_normal((B, nt, D))
    sv, sa = rng.integers(0, Cv, D), rng.integers(0, Ca, D)
    w_in = np.eye(Cv)[sv]          # row d picks channel sv[d]
    w_ain = np.eye(Ca)[sa]
    x = oe.embed_inputs(video, audio, text, L, w_in, np.zeros(D), w_ain, np.zeros(D), D)
    for b in range(B):
        for i, r in enumerate(L.video_indices):
            assert np.array_equal(x[b, r], video[b, i, sv])
        for j, r in enumerate(L.audio_indices):
            assert np.array_equal(x[b, r], audio[b, j, sa])
        for k, r in enumerate(L.text_indices):
            assert np.array_equal(x[b, r], text[b, k])
        pad = np.asarray(L.token_tags) == -1
        assert pad.sum() == 5 and np.all(x[b, pad] == 0.0)


def test_input_projection_matches_torch_linear_and_biases_land():
    dims, L = small_layout()
    rng = np.random.default_rng(2)
    D = dims.hidden
    video = rng.standard_normal((1, len(L.video_indices), 8))
    audio = rng.standard_normal((1, len(L.audio_indices), 4))
    text = rng.standard_normal((1, len(L.text_indices), D))
    w_in, b_in = rng.standard_normal((D, 8)), rng.standard_normal(D)
    w_ain, b_ain = rng.standard_normal((D, 4)), rng.standard_normal(D)
    x = oe.embed_inputs(video, audio, text, L, w_in, b_in, w_ain, b_ain, D)
    ref_v = F.linear(torch.from_numpy(video[0]), torch.from_numpy(w_in), torch.from_numpy(b_in)).numpy()
    ref_a = F.linear(torch.from_numpy(audio[0]), torch.from_numpy(w_ain), torch.from_numpy(b_ain)).numpy()
    close(x[0, L.video_indices], ref_v)
    close(x[0, L.audio_indices], ref_a)
    # zero latents leave exactly the biases
    z = oe.embed_inputs(0 * video, 0 * audio, text, L, w_in, b_in, w_ain, b_ain, D)
    close(z[0, L.video_indices], np.tile(b_in, (len(L.video_indices), 1)))


def test_norm_out_hand_worked_and_torch():
    # x = (1, 2, 3, 4), eps 0: mean 2.5, variance 1.25, so the normalised row
    # is (x - 2.5) / sqrt(1.25) = (-1.3416407864998738, -0.4472135954999579, ...);
    # with weight 2 and bias 1: (-1.6832815729997477, 0.10557280900008414, ...).
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    close(oe.norm_out(x, np.ones(4), np.zeros(4), 0.0),
          [[-1.3416407864998738, -0.4472135954999579, 0.4472135954999579, 1.3416407864998738]])
    close(oe.norm_out(x, np.full(4, 2.0), np.ones(4), 0.0),
          [[-1.6832815729997477, 0.10557280900008414, 1.8944271909999157, 3.6832815729997477]])
    rng = np.random.default_rng(3)
    y = rng.standard_normal((9, 48)) * 2 + 0.3
    g, b = rng.standard_normal(48), rng.standard_normal(48)
    ref = F.layer_norm(torch.from_numpy(y), (48,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5).numpy()
    close(oe.norm_out(y, g, b, 1e-5), ref)


def test_output_heads_gather_in_index_order_and_ignore_other_rows():
    dims, L = small_layout()
    rng = np.random.default_rng(4)
    B, D = 2, dims.hidden
    x = rng.standard_normal((B, L.seq_len, D))
    g, be = 1 + 0.1 * rng.standard_normal(D), 0.1 * rng.standard_normal(D)
    w_out, b_out = rng.standard_normal((6, D)), rng.standard_normal(6)
    w_aout, b_aout = rng.standard_normal((4, D)), rng.standard_normal(4)
    v, a = oe.output_heads(x, L, g, be, 1e-5, w_out, b_out, w_aout, b_aout)
    assert v.shape == (B, len(L.video_indices), 6) and a.shape == (B, len(L.audio_indices), 4)
    for b in range(B):
        hv = F.layer_norm(torch.from_numpy(x[b, L.video_indices]), (D,), torch.from_numpy(g), torch.from_numpy(be),
                          eps=1e-5)
        close(v[b], F.linear(hv, torch.from_numpy(w_out), torch.from_numpy(b_out)).numpy())
    # text and padding rows never reach the heads
    x2 = x.copy()
    other = np.setdiff1d(np.arange(L.seq_len), np.concatenate([L.video_indices, L.audio_indices]))
    x2[:, other] = 1e3 * rng.standard_normal((B, len(other), D))
    v2, a2 = oe.output_heads(x2, L, g, be, 1e-5, w_out, b_out, w_aout, b_aout)
    close(v2, v)
    close(a2, a)
    # the output follows the order of video_indices: reversing the index
    # tensor reverses the output rows
    L_rev = synth.Layout(L.token_tags, L.timestep_indices, L.position_ids, L.video_indices[::-1].copy(),
                         L.audio_indices, L.text_indices)
    v3, _ = oe.output_heads(x, L_rev, g, be, 1e-5, w_out, b_out, w_aout, b_aout)
    close(v3, v[:, ::-1])


def test_embed_then_heads_with_linear_weights_recovers_a_known_map():
    # With D = C_v, proj_in = identity (no bias) and norm_out weight 1 / bias 0,
    # the video head sees LayerNorm(video row): a closed form per row.
    dims = synth.ModelDims(hidden=8, num_heads=1, ffn_dim=8, num_tvals=2, dtype="f32")
    wl = synth.make_custom(dims, [("text", 2), ("audio", 3), ("video", 4, (1, 2, 2))], (1, 2, 2), 1, seed=5)
    L = wl.layout
    rng = np.random.default_rng(5)
    video = rng.standard_normal((1, 4, 8))
    x = oe.embed_inputs(video, rng.standard_normal((1, 3, 2)), rng.standard_normal((1, 2, 8)), L, np.eye(8),
                        np.zeros(8), rng.standard_normal((8, 2)), np.zeros(8), 8)
    v, _ = oe.output_heads(x, L, np.ones(8), np.zeros(8), 0.0, np.eye(8), np.zeros(8), np.zeros((2, 8)), np.zeros(2))
    mu = video.mean(-1, keepdims=True)
    sd = video.std(-1, keepdims=True)
    close(v, (video - mu) / sd)
