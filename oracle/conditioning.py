"""fp64 CPU oracle of the timestep conditioning that produces the per-block
AdaLN tables (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. It shares no code with the HIP path.

Sources:
  * page "MiniMaxH3Transformer3DModel", Parameters: freq_dim (width of the
    sinusoidal timestep embedding, timesteps taken unscaled in [0, 1]),
    time_embed_hidden_dim (inner width of the timestep MLP), time_embed_dim
    (its output width, the input of every AdaLN projection); the mixed
    precision note (the timestep MLP is float32, the block stack bfloat16);
    `forward`: `timestep` holds the distinct timestep values and
    `timestep_indices` points every row at one of them; the class
    description: the row's modality tag selects its AdaLN modulation.
  * page "HyperFlow for MiniMax-H3", How it works: the two-time embedder
    wraps the base timestep embedder, adds a copy for the step endpoint r
    and blends the two embeddings with a fixed gate; conditioning rows keep
    r = t.

The pages do not write the equations. Readings taken (one per function):
  a. sinusoid: half = freq_dim / 2 frequencies f_j = 10000^(-j / half),
     embedding [cos(t f_0..), sin(t f_0..)] (cosines first);
  b. timestep MLP: Linear(freq_dim -> hidden) with bias, SiLU,
     Linear(hidden -> embed) with bias;
  c. two-time blend: e = (1 - g) E(t) + g E'(r), E' an MLP of the same shape
     with its own weights (the base weights plus the merged adapter), g a
     scalar;
  d. AdaLN projection of tag k: table[k, v] = W_k SiLU(e_v) + b_k, a vector
     of 6 D values read as six rows of D in the order shift, scale, gate
     before attention, then shift, scale, gate before the FFN.
"""
from __future__ import annotations

import numpy as np

MAX_PERIOD = 10000.0


def sinusoid(t, freq_dim: int) -> np.ndarray:
    """[n] timesteps -> [n, freq_dim] embedding (reading a).

    Page "MiniMaxH3Transformer3DModel", Parameters, freq_dim: the timestep
    is used as given, in [0, 1], without a 1000x rescale.
    """
    t = np.asarray(t, np.float64).reshape(-1)
    half = freq_dim // 2
    freqs = np.exp(-np.log(MAX_PERIOD) * np.arange(half, dtype=np.float64) / half)
    ang = t[:, None] * freqs[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def time_mlp(s: np.ndarray, w1, b1, w2, b2) -> np.ndarray:
    """Timestep MLP (reading b): W2 SiLU(W1 s + b1) + b2, row by row.

    w1 [hidden, freq_dim], w2 [embed, hidden] (row-major [out, in]).
    """
    h = s @ np.asarray(w1, np.float64).T + np.asarray(b1, np.float64)
    return silu(h) @ np.asarray(w2, np.float64).T + np.asarray(b2, np.float64)


def time_embedding(t, freq_dim: int, base: dict, r=None, endpoint: dict = None, gate: float = 0.0) -> np.ndarray:
    """[n] timesteps -> [n, embed] time embeddings.

    base / endpoint: dicts with w1, b1, w2, b2. Without an endpoint embedder
    this is the base embedding E(t). With one (page "HyperFlow for
    MiniMax-H3", How it works) it is the blend of reading c,
    (1 - gate) E(t) + gate E'(r); r defaults to t, the conditioning rows'
    choice.
    """
    e_t = time_mlp(sinusoid(t, freq_dim), **base)
    if endpoint is None:
        return e_t
    r = t if r is None else r
    e_r = time_mlp(sinusoid(r, freq_dim), **endpoint)
    g = float(gate)
    return (1.0 - g) * e_t + g * e_r


def adaln_table(e: np.ndarray, w_proj: np.ndarray, b_proj, hidden: int) -> np.ndarray:
    """AdaLN table of one block (reading d).

    e [n, embed]; w_proj [tags, 6 D, embed]; b_proj [tags, 6 D] or None.
    Returns [tags, n, 6, D]: row (k, v) is tag k's projection of SiLU(e_v).
    """
    e = np.asarray(e, np.float64)
    w = np.asarray(w_proj, np.float64)
    T = w.shape[0]
    a = silu(e)
    out = np.empty((T, e.shape[0], 6, hidden))
    for k in range(T):
        y = a @ w[k].T
        if b_proj is not None:
            y = y + np.asarray(b_proj, np.float64)[k]
        out[k] = y.reshape(e.shape[0], 6, hidden)
    return out
