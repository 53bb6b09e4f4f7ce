"""Seeded synthetic workloads for the packed DiT block.

This module draws inputs only: layouts (row order, modality tags, timestep
indices, (t, h, w) positions, row-index tensors), latents, weights and AdaLN
tables. It holds none of the block's arithmetic, so both the fp64 oracle and
the HIP path can be fed from it. Every floating-point tensor that the HIP path
stores in bfloat16 is rounded here, once, to bfloat16 (round to nearest even),
and both sides receive those exact values.

The packed layout follows the MiniMaxH3Transformer3DModel page (class
description and `forward` parameters): one 1-D sequence holding text rows,
conditioning image/video rows, audio rows and target video rows, plus
optional padding rows (tag -1) that form their own attention document.

Recipe (per workload):
  * PRNG: ``numpy.random.default_rng(seed)`` (PCG64).
  * Draw order: pad count (multi-block workload only), timestep indices,
    latents, then per block: W_qkv, W_o, W_gate_up, W_down, g_q, g_k, table.
  * Row order: [text | conditioning | audio | target video | pad].
  * Tags: text 0, video 1 (conditioning rows included), audio 2, pad -1.
  * Positions: text row k -> (k, k, k); audio row a -> (a*T_v // n_audio, 0, 0)
    on the clock shared with the target video grid (T_v = its t extent);
    video rows -> row-major (t, h, w) over their grid; pad rows -> (0, 0, 0).
  * Timestep index uniform over [0, n_tvals) on real rows, 0 on pad rows.
  * Latents ~ N(0, 1); weights ~ N(0, 0.02); g_q, g_k = 1 + N(0, 0.02);
    table: all six modulation vectors (shift, scale, gate for attention and
    for the FFN) ~ N(0, 0.1) (fp32); gates near zero as in AdaLN-Zero, which
    keeps the block output at the scale its bf16 storage resolves.
  * Unit-gate variant (``gate_mean=1.0``): the same draws with 1 added to
    the two gate vectors, i.e. gates ~ N(1, 0.1). The branches then enter
    the output at full size and outputs reach |x| ~ 17, where one bf16 ulp
    is 0.125.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

TAG_TEXT, TAG_VIDEO, TAG_AUDIO, TAG_PAD = 0, 1, 2, -1
NUM_TAGS = 3


# --------------------------------------------------------------------------
# bfloat16 storage helpers (input preparation, shared by both sides)
# --------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A host tensor as the GPU will hold it.

    ``data`` is float32 (fp32 workloads) or uint16 bfloat16 bit patterns.
    ``values()`` widens the stored values exactly to float64.
    """
    data: np.ndarray
    dtype: str  # "bf16" | "f32"

    @property
    def shape(self):
        return self.data.shape

    def values(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)


def _normal(rng, shape, std, mean=0.0) -> np.ndarray:
    z = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        z *= np.float32(std)
    if mean != 0.0:
        z += np.float32(mean)
    return z


def _store(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        return Tensor(round_to_bf16_bits(x), "bf16")
    return Tensor(np.ascontiguousarray(x, dtype=np.float32), "f32")


# --------------------------------------------------------------------------
# Model / layout description
# --------------------------------------------------------------------------

@dataclasses.dataclass
class ModelDims:
    hidden: int = 5376
    num_heads: int = 56
    head_dim: int = 128
    ffn_dim: int = 14336
    rope_freq_dim: int = 16
    rope_theta: float = 1.0e4
    norm_eps: float = 1.0e-5
    qk_norm_eps: float = 1.0e-5
    num_tags: int = NUM_TAGS
    num_tvals: int = 8
    dtype: str = "bf16"  # activation + weight storage: "bf16" or "f32"

    @property
    def qkv_width(self) -> int:
        return self.num_heads * self.head_dim


@dataclasses.dataclass
class Layout:
    """One packed layout shared by every batch item."""
    token_tags: np.ndarray        # int32 [S]
    timestep_indices: np.ndarray  # int32 [S]
    position_ids: np.ndarray      # int32 [S, 3]
    video_indices: np.ndarray     # int32 [n_video]
    audio_indices: np.ndarray     # int32 [n_audio]
    text_indices: np.ndarray      # int32 [n_text]

    @property
    def seq_len(self) -> int:
        return int(self.token_tags.shape[0])

    @property
    def num_pad(self) -> int:
        return int((self.token_tags == TAG_PAD).sum())


@dataclasses.dataclass
class BlockWeights:
    w_qkv: Tensor      # [3W, D]
    w_out: Tensor      # [D, W]
    w_gate_up: Tensor  # [2F, D] rows [0,F) gate, [F,2F) up
    w_down: Tensor     # [D, F]
    q_norm: np.ndarray  # fp32 [hd]
    k_norm: np.ndarray  # fp32 [hd]
    adaln_table: np.ndarray  # fp32 [num_tags, num_tvals, 6, D]


@dataclasses.dataclass
class Workload:
    name: str
    dims: ModelDims
    layout: Layout
    x: Tensor                 # [B, S, D]
    blocks: List[BlockWeights]
    seed: int

    @property
    def batch(self) -> int:
        return int(self.x.shape[0])


# Segment kinds: ("text", n), ("audio", n), ("video", n, (t, h, w)) for the
# target grid and ("cond", n, (t, h, w)) for conditioning image/video rows.

def _grid_positions(n: int, grid: Tuple[int, int, int]) -> np.ndarray:
    t, h, w = grid
    r = np.arange(n, dtype=np.int64)
    if n <= t * h * w:
        return np.stack([r // (h * w), (r // w) % h, r % w], 1).astype(np.int32)
    # A single-frame grid listed with more rows than it holds: the extra rows
    # continue row-major past the last h row, (0, r // w, r % w).
    if t != 1:
        raise ValueError("only a single-frame grid may spill")
    return np.stack([np.zeros_like(r), r // w, r % w], 1).astype(np.int32)


def build_layout(segments, num_pad: int, target_grid: Tuple[int, int, int],
                 tidx: np.ndarray) -> Layout:
    """Lay rows out as [text | conditioning | audio | target video | pad]."""
    order = {"text": 0, "cond": 1, "audio": 2, "video": 3}
    segs = sorted(segments, key=lambda s: order[s[0]])
    tags, pos = [], []
    vid, aud, txt = [], [], []
    row = 0
    t_extent = target_grid[0]
    for seg in segs:
        kind = seg[0]
        if kind == "text":
            n = seg[1]
            k = np.arange(n, dtype=np.int32)
            pos.append(np.stack([k, k, k], 1))
            tags.append(np.full(n, TAG_TEXT, np.int32))
            txt.append(np.arange(row, row + n, dtype=np.int32))
        elif kind == "audio":
            n = seg[1]
            a = np.arange(n, dtype=np.int64)
            pt = (a * t_extent) // max(n, 1)
            pos.append(np.stack([pt, np.zeros_like(pt), np.zeros_like(pt)], 1).astype(np.int32))
            tags.append(np.full(n, TAG_AUDIO, np.int32))
            aud.append(np.arange(row, row + n, dtype=np.int32))
        elif kind in ("video", "cond"):
            n, grid = seg[1], seg[2]
            pos.append(_grid_positions(n, grid))
            tags.append(np.full(n, TAG_VIDEO, np.int32))
            vid.append(np.arange(row, row + n, dtype=np.int32))
        else:
            raise ValueError(kind)
        row += seg[1]
    if num_pad:
        pos.append(np.zeros((num_pad, 3), np.int32))
        tags.append(np.full(num_pad, TAG_PAD, np.int32))
    token_tags = np.concatenate(tags).astype(np.int32)
    S = token_tags.shape[0]
    assert tidx.shape == (S,)
    tidx = np.where(token_tags == TAG_PAD, 0, tidx).astype(np.int32)

    def cat(xs):
        return np.concatenate(xs).astype(np.int32) if xs else np.zeros(0, np.int32)

    return Layout(token_tags, tidx, np.concatenate(pos).astype(np.int32),
                  cat(vid), cat(aud), cat(txt))


GATE_SLOTS = (2, 5)  # gate vectors of the attention and FFN residuals in a table entry


def draw_block(rng, dims: ModelDims, gate_mean: float = 0.0) -> BlockWeights:
    D, W, F, hd = dims.hidden, dims.qkv_width, dims.ffn_dim, dims.head_dim
    w_qkv = _store(_normal(rng, (3 * W, D), 0.02), dims.dtype)
    w_out = _store(_normal(rng, (D, W), 0.02), dims.dtype)
    w_gate_up = _store(_normal(rng, (2 * F, D), 0.02), dims.dtype)
    w_down = _store(_normal(rng, (D, F), 0.02), dims.dtype)
    q_norm = _normal(rng, (hd,), 0.02, 1.0)
    k_norm = _normal(rng, (hd,), 0.02, 1.0)
    table = _normal(rng, (dims.num_tags, dims.num_tvals, 6, D), 0.1)
    if gate_mean:
        table[:, :, list(GATE_SLOTS)] += np.float32(gate_mean)
    return BlockWeights(w_qkv, w_out, w_gate_up, w_down, q_norm, k_norm, table)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------

WORKLOADS = {
    # hidden 512, 4 x 128 heads, FFN 1024, fp32; 48 text, 16 audio,
    # 240 video on (4, 6, 10), 16 pads: 320 rows.
    "tiny": dict(dims=dict(hidden=512, num_heads=4, head_dim=128, ffn_dim=1024, dtype="f32"),
                 segments=[("text", 48), ("audio", 16), ("video", 240, (4, 6, 10))],
                 target_grid=(4, 6, 10), pads=16, n_tvals=8, blocks=1),
    # full width, padless: 512 text, 256 audio, 7424 video on (4, 32, 58).
    "padless8k": dict(dims=dict(), segments=[("text", 512), ("audio", 256), ("video", 7424, (4, 32, 58))],
                      target_grid=(4, 32, 58), pads=0, n_tvals=8, blocks=1),
    # full width with padding: 1024 text, 512 conditioning-image rows on
    # (1, 24, 21) (24*21 = 504, so the last 8 rows spill into h = 24),
    # 768 audio, 13440 video on (10, 24, 56), 640 pads.
    "padded16k": dict(dims=dict(), segments=[("text", 1024), ("cond", 512, (1, 24, 21)), ("audio", 768),
                                             ("video", 13440, (10, 24, 56))],
                      target_grid=(10, 24, 56), pads=640, n_tvals=8, blocks=1),
    # clip scale: 1024 text, 1536 audio, 30208 video on (16, 32, 59); the
    # timestep index enumerates (sigma_now, sigma_next) pairs on an 8-point grid.
    "clip32k": dict(dims=dict(), segments=[("text", 1024), ("audio", 1536), ("video", 30208, (16, 32, 59))],
                    target_grid=(16, 32, 59), pads=0, n_tvals=64, blocks=1),
    # four chained blocks: 2048 text, 3072 conditioning video on (2, 24, 64),
    # 1024 audio, 18432 video on (12, 24, 64), and 0-1023 pads drawn from the seed.
    "chain4x24k": dict(dims=dict(), segments=[("text", 2048), ("cond", 3072, (2, 24, 64)), ("audio", 1024),
                                              ("video", 18432, (12, 24, 64))],
                       target_grid=(12, 24, 64), pads="seeded", n_tvals=8, blocks=4),
}

WORKLOAD_ORDER = ["tiny", "padless8k", "padded16k", "clip32k", "chain4x24k"]


def workload_dims(name: str) -> ModelDims:
    spec = WORKLOADS[name]
    return ModelDims(num_tvals=spec["n_tvals"], **spec["dims"])


def make_workload(name: str, seed: int = 0, batch: int = 1, with_weights: bool = True,
                  num_blocks: Optional[int] = None, gate_mean: float = 0.0) -> Workload:
    spec = WORKLOADS[name]
    dims = workload_dims(name)
    rng = np.random.default_rng(seed)
    pads = spec["pads"]
    if pads == "seeded":
        pads = int(rng.integers(0, 1024))
    n_real = sum(s[1] for s in spec["segments"])
    S = n_real + pads
    tidx = rng.integers(0, dims.num_tvals, size=S).astype(np.int32)
    layout = build_layout(spec["segments"], pads, spec["target_grid"], tidx)
    x = _store(_normal(rng, (batch, S, dims.hidden), 1.0), dims.dtype)
    nb = spec["blocks"] if num_blocks is None else num_blocks
    blocks = [draw_block(rng, dims, gate_mean) for _ in range(nb)] if with_weights else []
    return Workload(name, dims, layout, x, blocks, seed)


def make_custom(dims: ModelDims, segments, target_grid, pads: int, seed: int = 0, batch: int = 1,
                num_blocks: int = 1) -> Workload:
    """A small workload of any shape, drawn with the same recipe."""
    rng = np.random.default_rng(seed)
    n_real = sum(s[1] for s in segments)
    S = n_real + pads
    tidx = rng.integers(0, dims.num_tvals, size=S).astype(np.int32)
    layout = build_layout(segments, pads, target_grid, tidx)
    x = _store(_normal(rng, (batch, S, dims.hidden), 1.0), dims.dtype)
    blocks = [draw_block(rng, dims) for _ in range(num_blocks)]
    return Workload("custom", dims, layout, x, blocks, seed)


def permute_rows(layout: Layout, perm: np.ndarray) -> Layout:
    """Reorder packed rows: new row i is old row perm[i]; index tensors follow."""
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.shape[0])
    return Layout(layout.token_tags[perm].copy(), layout.timestep_indices[perm].copy(),
                  layout.position_ids[perm].copy(), inv[layout.video_indices].astype(np.int32),
                  inv[layout.audio_indices].astype(np.int32), inv[layout.text_indices].astype(np.int32))


# --------------------------------------------------------------------------
# Timestep conditioning inputs (the AdaLN table build)
# --------------------------------------------------------------------------
#
# Recipe: ``numpy.random.default_rng(seed)``; draw order: base embedder
# (W1, b1, W2, b2), endpoint embedder (same order, two-time only), then per
# block the AdaLN projection (W, b). Embedder weights are fp32 with
# W ~ N(0, 1 / fan_in) and biases ~ N(0, 0.02); the endpoint embedder is the
# base one plus N(0, 0.1^2 / fan_in) (a merged adapter); gate 0.25. AdaLN
# projection weights and biases ~ N(0, 0.02) in the activation dtype.
# Timesteps: value v of n is 1 - v / n; with two-time conditioning over
# n = k * k values, value v is the pair (t, r) = (g[v // k], g[v % k]) on the
# k-point grid g_i = 1 - i / k, so the diagonal holds the r = t pairs.

@dataclasses.dataclass
class TimeEmbedder:
    w1: np.ndarray  # fp32 [hidden_dim, freq_dim]
    b1: np.ndarray  # fp32 [hidden_dim]
    w2: np.ndarray  # fp32 [embed_dim, hidden_dim]
    b2: np.ndarray  # fp32 [embed_dim]

    def as_dict(self) -> dict:
        return dict(w1=self.w1, b1=self.b1, w2=self.w2, b2=self.b2)


@dataclasses.dataclass
class Conditioning:
    freq_dim: int
    hidden_dim: int
    embed_dim: int
    t: np.ndarray                   # fp32 [n_tvals]
    r: Optional[np.ndarray]         # fp32 [n_tvals] step endpoints (two-time only)
    base: TimeEmbedder
    endpoint: Optional[TimeEmbedder]
    gate: float
    w_proj: List[Tensor]            # per block [num_tags, 6 D, embed_dim]
    b_proj: List[Tensor]            # per block [num_tags, 6 D]


def _draw_embedder(rng, freq_dim, hidden_dim, embed_dim) -> TimeEmbedder:
    return TimeEmbedder(_normal(rng, (hidden_dim, freq_dim), freq_dim ** -0.5), _normal(rng, (hidden_dim,), 0.02),
                        _normal(rng, (embed_dim, hidden_dim), hidden_dim ** -0.5), _normal(rng, (embed_dim,), 0.02))


def make_conditioning(dims: ModelDims, num_blocks: int = 1, two_time: bool = False, seed: int = 0,
                      freq_dim: int = 256, hidden_dim: int = 5376, embed_dim: int = 2688,
                      num_tvals: Optional[int] = None) -> Conditioning:
    """Timesteps, timestep-MLP weights and per-block AdaLN projections."""
    rng = np.random.default_rng(seed)
    n = dims.num_tvals if num_tvals is None else num_tvals
    base = _draw_embedder(rng, freq_dim, hidden_dim, embed_dim)
    endpoint, r = None, None
    if two_time:
        k = int(round(n ** 0.5))
        if k * k != n:
            raise ValueError("two-time conditioning needs a square number of timestep values")
        d = _draw_embedder(rng, freq_dim, hidden_dim, embed_dim)
        endpoint = TimeEmbedder(base.w1 + np.float32(0.1) * d.w1, base.b1.copy(),
                                base.w2 + np.float32(0.1) * d.w2, base.b2.copy())
        g = (1.0 - np.arange(k) / k).astype(np.float32)
        v = np.arange(n)
        t, r = g[v // k], g[v % k]
    else:
        t = (1.0 - np.arange(n) / n).astype(np.float32)
    D6 = 6 * dims.hidden
    w_proj, b_proj = [], []
    for _ in range(num_blocks):
        w_proj.append(_store(_normal(rng, (dims.num_tags, D6, embed_dim), 0.02), dims.dtype))
        b_proj.append(_store(_normal(rng, (dims.num_tags, D6), 0.02), dims.dtype))
    return Conditioning(freq_dim, hidden_dim, embed_dim, np.asarray(t, np.float32),
                        None if r is None else np.asarray(r, np.float32), base, endpoint,
                        0.25 if two_time else 0.0, w_proj, b_proj)


# --------------------------------------------------------------------------
# Model edges: latent rows and the input / output projections
# --------------------------------------------------------------------------
#
# Recipe: ``numpy.random.default_rng(seed)``; draw order: video latent rows
# [B, n_video, 96], audio latent rows [B, n_audio, 32], embedded text rows
# [B, n_text, D] (activation dtype), then proj_in W [D, 96] and b,
# audio_proj_in W [D, 32] and b, norm_out weight and bias, proj_out W [96, D]
# and b, audio_proj_out W [32, D] and b. Latents N(0, 1); projection weights
# N(0, 1 / fan_in), biases N(0, 0.02); norm_out weight 1 + N(0, 0.02), bias
# N(0, 0.02). Everything but the text rows is fp32.

@dataclasses.dataclass
class Edges:
    video: np.ndarray      # fp32 [B, n_video, C_v]
    audio: np.ndarray      # fp32 [B, n_audio, C_a]
    text: Tensor           # [B, n_text, D] activation dtype
    w_in: np.ndarray       # fp32 [D, C_v]
    b_in: np.ndarray       # fp32 [D]
    w_ain: np.ndarray      # fp32 [D, C_a]
    b_ain: np.ndarray      # fp32 [D]
    gamma: np.ndarray      # fp32 [D]
    beta: np.ndarray       # fp32 [D]
    w_out: np.ndarray      # fp32 [C_v, D]
    b_out: np.ndarray      # fp32 [C_v]
    w_aout: np.ndarray     # fp32 [C_a, D]
    b_aout: np.ndarray     # fp32 [C_a]
    final_norm_eps: float = 1.0e-5


def make_edges(dims: ModelDims, layout: Layout, batch: int = 1, seed: int = 0, video_channels: int = 96,
               audio_channels: int = 32) -> Edges:
    rng = np.random.default_rng(seed)
    D = dims.hidden
    nv, na, nt = (int(layout.video_indices.shape[0]), int(layout.audio_indices.shape[0]),
                  int(layout.text_indices.shape[0]))
    video = _normal(rng, (batch, nv, video_channels), 1.0)
    audio = _normal(rng, (batch, na, audio_channels), 1.0)
    text = _store(_normal(rng, (batch, nt, D), 1.0), dims.dtype)
    w_in = _normal(rng, (D, video_channels), video_channels ** -0.5)
    b_in = _normal(rng, (D,), 0.02)
    w_ain = _normal(rng, (D, audio_channels), audio_channels ** -0.5)
    b_ain = _normal(rng, (D,), 0.02)
    gamma = _normal(rng, (D,), 0.02, 1.0)
    beta = _normal(rng, (D,), 0.02)
    w_out = _normal(rng, (video_channels, D), D ** -0.5)
    b_out = _normal(rng, (video_channels,), 0.02)
    w_aout = _normal(rng, (audio_channels, D), D ** -0.5)
    b_aout = _normal(rng, (audio_channels,), 0.02)
    return Edges(video, audio, text, w_in, b_in, w_ain, b_ain, gamma, beta, w_out, b_out, w_aout, b_aout)


# --------------------------------------------------------------------------
# Unmerged adapters of the block projections
# --------------------------------------------------------------------------
#
# Recipe: ``numpy.random.default_rng(seed)``; per block, for the projections
# qkv, out, gate_up, down in that order: A [rank, K] ~ N(0, 1 / K), then
# B [N, rank] ~ N(0, 0.02^2), both in the activation dtype. (A trained
# adapter starts from B = 0; a random B makes the low-rank path visible.)

LORA_SHAPES = ("qkv", "out", "gate_up", "down")


def lora_shapes(dims: ModelDims) -> dict:
    """(N, K) of each projection's base weight."""
    D, W, F = dims.hidden, dims.qkv_width, dims.ffn_dim
    return {"qkv": (3 * W, D), "out": (D, W), "gate_up": (2 * F, D), "down": (D, F)}


def make_lora(dims: ModelDims, rank: int, num_blocks: int = 1, seed: int = 0) -> List[dict]:
    """Per block {name: (A, B)} as stored Tensors."""
    rng = np.random.default_rng(seed)
    shapes = lora_shapes(dims)
    out = []
    for _ in range(num_blocks):
        blk = {}
        for n in LORA_SHAPES:
            N, K = shapes[n]
            a = _store(_normal(rng, (rank, K), K ** -0.5), dims.dtype)
            b = _store(_normal(rng, (N, rank), 0.02), dims.dtype)
            blk[n] = (a, b)
        out.append(blk)
    return out


def make_time_lora(cond: "Conditioning", rank: int, seed: int = 0) -> List[dict]:
    """Adapters of the timestep MLPs (base, then endpoint when present), fp32:
    A1 [rank, freq] ~ N(0, 1 / freq), B1 [hidden, rank] ~ N(0, 0.02^2),
    A2 [rank, hidden] ~ N(0, 1 / hidden), B2 [embed, rank] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    F, Hd, E = cond.freq_dim, cond.hidden_dim, cond.embed_dim
    out = []
    for _ in range(2 if cond.endpoint is not None else 1):
        out.append(dict(a1=_normal(rng, (rank, F), F ** -0.5), b1=_normal(rng, (Hd, rank), 0.02),
                        a2=_normal(rng, (rank, Hd), Hd ** -0.5), b2=_normal(rng, (E, rank), 0.02)))
    return out
