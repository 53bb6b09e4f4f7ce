"""fp64 CPU oracle of the model's edges around the block stack: the input
projections that build the packed sequence and the output heads that read it
back (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. It shares no code with the HIP path.

Source: page "MiniMaxH3Transformer3DModel": Parameters in_channels (24),
patch_size ((1, 2, 2)), audio_in_channels (32), hidden_size, final_norm_eps
(the eps of norm_out); the mixed-precision note (the two input patch
projections and the two output heads are float32); `forward`: the video rows
arrive patchified, in_channels * prod(patch_size) wide, in the order of
video_indices, the audio rows in the order of audio_indices; the outputs are
the video and audio velocities in those same row orders. Module names
proj_in, audio_proj_in, norm_out, proj_out, audio_proj_out appear in the
page's quantization example.

Readings (the pages name the parts, not their equations):
  a. proj_in / audio_proj_in: Linear with bias from the latent width to the
     hidden size; row i of the video input lands on packed row
     video_indices[i], row j of the audio input on audio_indices[j];
  b. text rows arrive already embedded (hidden-size wide) and are copied to
     text_indices (the text refiner is outside this path); rows no index
     tensor addresses (padding) are zero;
  c. norm_out: LayerNorm over the hidden size with final_norm_eps and a
     learned weight and bias, shared by the video and audio rows;
  d. proj_out / audio_proj_out: Linear with bias back to the latent widths,
     applied to norm_out of the rows at video_indices / audio_indices, in
     that order.
"""
from __future__ import annotations

import numpy as np


def embed_inputs(video, audio, text, layout, w_in, b_in, w_ain, b_ain, hidden: int) -> np.ndarray:
    """Packed sequence [B, S, D] from the video [B, n_v, C_v], audio
    [B, n_a, C_a] and (embedded) text [B, n_t, D] rows (readings a, b)."""
    video = np.asarray(video, np.float64)
    B = video.shape[0]
    S = int(np.asarray(layout.token_tags).shape[0])
    x = np.zeros((B, S, hidden))
    vi = np.asarray(layout.video_indices, np.int64)
    ai = np.asarray(layout.audio_indices, np.int64)
    ti = np.asarray(layout.text_indices, np.int64)
    x[:, vi] = video @ np.asarray(w_in, np.float64).T + np.asarray(b_in, np.float64)
    x[:, ai] = np.asarray(audio, np.float64) @ np.asarray(w_ain, np.float64).T + np.asarray(b_ain, np.float64)
    x[:, ti] = np.asarray(text, np.float64)
    return x


def norm_out(x: np.ndarray, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with weight and bias (reading c)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def output_heads(x, layout, gamma, beta, eps, w_out, b_out, w_aout, b_aout):
    """(video velocity [B, n_v, C_v], audio velocity [B, n_a, C_a]) from the
    final packed hidden states x [B, S, D] (readings c, d)."""
    x = np.asarray(x, np.float64)
    vi = np.asarray(layout.video_indices, np.int64)
    ai = np.asarray(layout.audio_indices, np.int64)
    hv = norm_out(x[:, vi], gamma, beta, eps)
    ha = norm_out(x[:, ai], gamma, beta, eps)
    v = hv @ np.asarray(w_out, np.float64).T + np.asarray(b_out, np.float64)
    a = ha @ np.asarray(w_aout, np.float64).T + np.asarray(b_aout, np.float64)
    return v, a
