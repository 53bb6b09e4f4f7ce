"""fp64 CPU oracle of one packed DiT block forward (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. It shares no code with the HIP path.

What it computes follows the MiniMaxH3Transformer3DModel page (diffusers API
documentation: class description, Parameters, `forward`). The page names the
parts of a block but never writes its equations; where it is silent the
plainest reading is taken, and each such reading is stated at the function
that depends on it:

  1. per-row AdaLN before attention: non-affine LayerNorm (norm_eps), then
     (1 + scale) and shift chosen by the row's (modality tag, timestep index);
  2. QKV projection, hidden -> 3 x (num_heads x head_dim), no bias;
  3. per-head RMSNorm of q and k (qk_norm_eps, one weight of length head_dim);
  4. 3-D rotary embedding on 2*3*rope_freq_dim channels;
  5. full self-attention; padding rows (tag -1) form their own document;
  6. output projection, added to the residual scaled by the AdaLN gate;
  7. per-row AdaLN before the FFN, SwiGLU FFN, gated residual.

Everything is float64; tensors arrive as the exact values the GPU stores.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from typing import Dict, Optional, Sequence

import numpy as np

TAG_PAD = -1


# --------------------------------------------------------------------------
# 1 / 7: AdaLN modulation selected per row
# --------------------------------------------------------------------------

def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Non-affine LayerNorm over the last axis: mean and biased variance.

    Reading: the page gives only the eps of the pre-attention and pre-FFN
    norms (Parameters: norm_eps); as the modulation supplies the affine
    part, the norm itself carries no weight or bias.
    """
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulation(table: np.ndarray, tags: np.ndarray, tidx: np.ndarray, which: int):
    """(shift, scale, gate) for every row, each [S, D].

    The row's modality tag selects the AdaLN parameters (class description);
    the timestep index picks the row's noise level (`forward`:
    timestep_indices). Reading: table[tag, tidx] holds six vectors, shift,
    scale, gate for attention (which=0) then for the FFN (which=1). Padding
    rows have no table entry: their shift, scale and gate are zero.
    """
    S = tags.shape[0]
    D = table.shape[-1]
    shift = np.zeros((S, D))
    scale = np.zeros((S, D))
    gate = np.zeros((S, D))
    real = tags != TAG_PAD
    sel = table[tags[real], tidx[real]].astype(np.float64)  # [n_real, 6, D]
    shift[real] = sel[:, 3 * which + 0]
    scale[real] = sel[:, 3 * which + 1]
    gate[real] = sel[:, 3 * which + 2]
    return shift, scale, gate


def adaln(x: np.ndarray, table, tags, tidx, which: int, eps: float) -> np.ndarray:
    """LN(x) * (1 + scale) + shift, per row."""
    shift, scale, _ = modulation(table, tags, tidx, which)
    return layer_norm(x, eps) * (1.0 + scale) + shift


# --------------------------------------------------------------------------
# 3: per-head query / key RMSNorm
# --------------------------------------------------------------------------

def rms_norm_heads(q: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """q [..., H, hd] -> q * g / sqrt(mean(q^2) + eps) over hd.

    Reading: "per-head query/key norms" (Parameters: qk_norm_eps) is an
    RMSNorm whose weight of length head_dim is shared by all heads.
    """
    ms = (q ** 2).mean(axis=-1, keepdims=True)
    return q * np.asarray(g, np.float64) / np.sqrt(ms + eps)


# --------------------------------------------------------------------------
# 4: 3-D rotary embedding
# --------------------------------------------------------------------------

def rope_inv_freq(freq_dim: int, theta: float) -> np.ndarray:
    """The inv_freq buffer shared by the t, h and w axes.

    Reading: the usual schedule for a rotary block of 2*freq_dim channels,
    theta ** (-2j / (2*freq_dim)) = theta ** (-j / freq_dim), j < freq_dim
    (Parameters: rope_freq_dim, rope_theta).
    """
    j = np.arange(freq_dim, dtype=np.float64)
    return np.power(float(theta), -j / freq_dim)


def rope_3d(q: np.ndarray, pos: np.ndarray, freq_dim: int, theta: float) -> np.ndarray:
    """Rotate q [S, H, hd] by the row positions pos [S, 3] = (t, h, w).

    2*3*freq_dim channels are rotated (Parameters: rope_freq_dim). Reading:
    axis a in {t, h, w} owns channels [2*freq_dim*a, 2*freq_dim*(a+1)), its
    pair j is channels (2j, 2j+1) inside that block, rotated by the angle
    pos[a] * inv_freq[j]; the remaining channels pass through unchanged.
    """
    out = np.array(q, dtype=np.float64, copy=True)
    inv_freq = rope_inv_freq(freq_dim, theta)
    for a in range(3):
        ang = pos[:, a].astype(np.float64)[:, None] * inv_freq[None, :]  # [S, fd]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        base = 2 * freq_dim * a
        u = q[:, :, base + 0: base + 2 * freq_dim: 2]
        v = q[:, :, base + 1: base + 2 * freq_dim: 2]
        out[:, :, base + 0: base + 2 * freq_dim: 2] = u * c - v * s
        out[:, :, base + 1: base + 2 * freq_dim: 2] = u * s + v * c
    return out


# --------------------------------------------------------------------------
# 5: attention with padding rows in their own document
# --------------------------------------------------------------------------

def attention_doc_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, doc: np.ndarray,
                         scale: float, rows: Optional[np.ndarray] = None,
                         chunk: int = 1024, threads: Optional[int] = None) -> np.ndarray:
    """o_i = sum_j softmax_j(q_i . k_j * scale) v_j over j with doc(j) == doc(i).

    Full self-attention over the packed sequence (class description); rows
    whose tag is -1 form their own attention document via a boolean mask.
    q, k, v: [S, H, hd]. ``rows`` restricts the queries (all keys are used);
    the result is [len(rows), H, hd]. Two-pass softmax per query chunk:
    max, exp, sum, normalise.
    """
    S, H, hd = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty((rows.shape[0], H, hd))

    def one_head(h):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for c0 in range(0, rows.shape[0], chunk):
            r = rows[c0:c0 + chunk]
            s = (q[r, h, :] @ kh.T) * scale                      # [n, S]
            allowed = doc[r][:, None] == doc[None, :]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            out[c0:c0 + chunk, h, :] = p @ vh

    n_threads = threads or min(H, os.cpu_count() or 1)
    if n_threads <= 1 or S * rows.shape[0] < (1 << 22):
        for h in range(H):
            one_head(h)
    else:
        # heads run in parallel threads, each with a single-threaded BLAS
        try:
            from threadpoolctl import threadpool_limits
            limit = threadpool_limits(limits=1, user_api="blas")
        except ImportError:  # pragma: no cover
            limit = None
        try:
            with cf.ThreadPoolExecutor(n_threads) as ex:
                list(ex.map(one_head, range(H)))
        finally:
            if limit is not None:
                limit.restore_original_limits()
    return out


def doc_ids(tags: np.ndarray) -> np.ndarray:
    """Attention document of each row: 1 for padding rows (tag -1), else 0."""
    return (np.asarray(tags) == TAG_PAD).astype(np.int64)


# --------------------------------------------------------------------------
# 8: SwiGLU
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(b: np.ndarray, w_gate_up: np.ndarray, ffn_dim: int) -> np.ndarray:
    """silu(b W_gate^T) * (b W_up^T), W_gate = rows [0, F), W_up = rows [F, 2F).

    Reading: "SwiGLU feed-forward" of inner width ffn_dim (Parameters).
    """
    g = b @ w_gate_up[:ffn_dim].T
    u = b @ w_gate_up[ffn_dim:].T
    return silu(g) * u


# --------------------------------------------------------------------------
# The block
# --------------------------------------------------------------------------

def block_forward(x: np.ndarray, layout, w: Dict[str, np.ndarray], dims,
                  rows: Optional[Sequence[int]] = None, taps: bool = False):
    """One block over one packed sequence; x [S, D] float64.

    ``w`` holds float64 w_qkv [3W, D], w_out [D, W], w_gate_up [2F, D],
    w_down [D, F], q_norm [hd], k_norm [hd] and adaln_table
    [tags, tvals, 6, D]. ``rows``: compute the output for these query rows
    only (keys and values still come from every row). Returns the output
    rows, or (output, taps dict) with ``taps=True``.
    """
    tags = np.asarray(layout.token_tags)
    tidx = np.asarray(layout.timestep_indices)
    pos = np.asarray(layout.position_ids)
    S, D = x.shape
    H, hd, F = dims.num_heads, dims.head_dim, dims.ffn_dim
    W = H * hd
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    table = w["adaln_table"]

    # 1. AdaLN before attention (all rows: every row is a key/value)
    a = adaln(x, table, tags, tidx, 0, dims.norm_eps)
    # 2. projections: keys/values for every row, queries for the output rows
    wq, wk, wv = w["w_qkv"][:W], w["w_qkv"][W:2 * W], w["w_qkv"][2 * W:]
    q = (a[rows] @ wq.T).reshape(len(rows), H, hd)
    k = (a @ wk.T).reshape(S, H, hd)
    v = (a @ wv.T).reshape(S, H, hd)
    # 3. per-head RMSNorm, 4. rotary embedding
    qn = rope_3d(rms_norm_heads(q, w["q_norm"], dims.qk_norm_eps), pos[rows],
                 dims.rope_freq_dim, dims.rope_theta)
    kn = rope_3d(rms_norm_heads(k, w["k_norm"], dims.qk_norm_eps), pos,
                 dims.rope_freq_dim, dims.rope_theta)
    # 5. attention (queries `rows`, keys/values all rows)
    doc = doc_ids(tags)
    q_full = np.zeros((S, H, hd))
    q_full[rows] = qn
    o = attention_doc_masked(q_full, kn, v, doc, 1.0 / np.sqrt(hd), rows=rows)
    o = o.reshape(len(rows), W)
    # 6. output projection + gated residual
    x_r = x[rows]
    _, _, gate1 = modulation(table, tags[rows], tidx[rows], 0)
    attn_proj = o @ w["w_out"].T
    x_mid = x_r + gate1 * attn_proj
    # 7. AdaLN before the FFN, SwiGLU, gated residual
    b = adaln(x_mid, table, tags[rows], tidx[rows], 1, dims.norm_eps)
    h = swiglu(b, w["w_gate_up"], F)
    _, _, gate2 = modulation(table, tags[rows], tidx[rows], 1)
    ffn_out = h @ w["w_down"].T
    out = x_mid + gate2 * ffn_out
    if not taps:
        return out
    return out, dict(adaln1=a[rows], q_rot=qn, k_rot=kn[rows], v=v[rows], attn_o=o,
                     attn_proj=attn_proj, x_mid=x_mid, adaln2=b, ffn_h=h, ffn_out=ffn_out)


def chain_forward(x: np.ndarray, layout, blocks: Sequence[Dict[str, np.ndarray]], dims,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Blocks applied in sequence (a stack of blocks, Parameters: num_layers).

    Every block but the last runs on all rows; the last may be restricted
    to ``rows``.
    """
    for i, w in enumerate(blocks):
        last = i == len(blocks) - 1
        x = block_forward(x, layout, w, dims, rows=rows if last else None)
    return x


def block_forward_batched(x: np.ndarray, layout, w, dims, rows=None) -> np.ndarray:
    """x [B, S, D]: every batch item is its own sequence sharing one layout
    (the batch axis is a pure replication axis, class description)."""
    return np.stack([block_forward(x[b], layout, w, dims, rows=rows) for b in range(x.shape[0])])
