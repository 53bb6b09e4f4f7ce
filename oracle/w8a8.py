"""CPU oracle of the rotated W8A8 INT8 linear layer (TEST INFRASTRUCTURE
ONLY).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. It shares no code with the HIP path.

Source: page "HyperFlow H3 Flash Brings MiniMax H3 Video to One GPU", How it
got smaller and faster: rotated W8A8 INT8 quantization of 180 linear layers
(8-bit integer weights and activations). The page names the technique, not
its form. Readings:
  a. rotation: the block-diagonal normalised Hadamard transform over the
     input dimension in blocks of 128, applied to the activations and to the
     weight rows alike, so that (x H)(W H)^T = x W^T (H H^T = I);
  b. quantization: symmetric int8 per row (per token for activations, per
     output channel for weights): amax = max |v|, code = rint(v * (127 /
     amax)) in [-127, 127], scale = amax / 127; an all-zero row has codes 0
     and scale 0;
  c. the product: exact int32 accumulation of the codes, then
     y = acc * scale_x * scale_w.
The codes are integers decided by floating point, so the rotation and the
quantization are computed in float32, in the order stated at each function
(the GPU path takes the same decisions in the same precision); the product
is exact in integers and its dequantization is evaluated in float64.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
# 1 / sqrt(128) rounded to float32
INV_SQRT_BLOCK = np.float32(1.0 / np.sqrt(128.0))


def fwht_blocks_f32(x) -> np.ndarray:
    """Normalised Hadamard transform of every 128-wide block of the last axis
    (reading a), in float32: butterfly stages h = 1, 2, 4, ..., 64, each
    mapping the pair (i, i + h) (bit h of i clear) to (x_i + x_{i+h},
    x_i - x_{i+h}), then one multiplication by 1/sqrt(128)."""
    v = np.array(x, dtype=np.float32, copy=True)
    K = v.shape[-1]
    assert K % BLOCK == 0
    lead = v.shape[:-1]
    v = v.reshape(-1, K // BLOCK, BLOCK)
    h = 1
    while h < BLOCK:
        w = v.reshape(v.shape[0], v.shape[1], BLOCK // (2 * h), 2, h)
        a = w[:, :, :, 0, :].copy()
        b = w[:, :, :, 1, :].copy()
        w[:, :, :, 0, :] = a + b
        w[:, :, :, 1, :] = a - b
        h *= 2
    v = v * INV_SQRT_BLOCK
    return v.reshape(*lead, K)


def quantize_rows_f32(v):
    """Symmetric per-row int8 quantization (reading b) of float32 rows:
    returns (codes int8, scale float32)."""
    v = np.asarray(v, np.float32)
    amax = np.abs(v).max(axis=-1)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(127.0) / safe).astype(np.float32)
    q = np.rint(v * inv[..., None]).astype(np.float32)
    q = np.clip(q, -127, 127)
    q = np.where(amax[..., None] > 0, q, 0).astype(np.int8)
    scale = np.where(amax > 0, amax / np.float32(127.0), np.float32(0.0)).astype(np.float32)
    return q, scale


def rotate_quantize(x):
    """Rotation then quantization of rows (activations or weight rows)."""
    return quantize_rows_f32(fwht_blocks_f32(np.asarray(x, np.float32)))


def int_matmul(qa, qw) -> np.ndarray:
    """Exact integer product qa [M, K] . qw [N, K]^T (reading c), int64.

    Evaluated as a float64 product: every term is at most 127^2 and every
    partial sum at most K * 127^2 < 2^53, so each float64 operation is exact.
    """
    qa, qw = np.asarray(qa), np.asarray(qw)
    assert qa.shape[-1] * 127 * 127 < 2 ** 53
    return (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def linear_w8a8(x, w) -> np.ndarray:
    """y = x W^T through the rotated W8A8 path, dequantized in float64."""
    qx, sx = rotate_quantize(x)
    qw, sw = rotate_quantize(w)
    acc = int_matmul(qx, qw).astype(np.float64)
    return acc * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]


# --------------------------------------------------------------------------
# A block with every projection on rotated W8A8
# --------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """float64 -> float32 -> bfloat16 (round to nearest even) -> float64: the
    value a bf16 activation tensor holds."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def block_forward_w8a8(x, layout, w, dims, taps: bool = False):
    """One block (the steps of oracle.block.block_forward) with each of the
    four projections on rotated W8A8. A bf16 block feeds its projections
    bf16 tensors, so each input (the AdaLN outputs, the attention output, the
    SwiGLU output) is rounded to bf16 before it is rotated and quantized;
    the weights are the block's bf16 matrices, rotated and quantized per row.
    With ``taps`` returns (output, dict) with the four projection inputs as
    rounded to bf16 (adaln1, attn_o, adaln2, ffn_h) and the products of the
    output and down projections (attn_proj, ffn_out)."""
    from . import block as ob
    tags = np.asarray(layout.token_tags)
    tidx = np.asarray(layout.timestep_indices)
    pos = np.asarray(layout.position_ids)
    S, D = x.shape
    H, hd, F = dims.num_heads, dims.head_dim, dims.ffn_dim
    W = H * hd
    table = w["adaln_table"]

    def lin(inp, wm):
        return linear_w8a8(round_bf16(inp), wm)

    a = ob.adaln(x, table, tags, tidx, 0, dims.norm_eps)
    qkv = lin(a, w["w_qkv"])
    q = qkv[:, :W].reshape(S, H, hd)
    k = qkv[:, W:2 * W].reshape(S, H, hd)
    v = qkv[:, 2 * W:].reshape(S, H, hd)
    qn = ob.rope_3d(ob.rms_norm_heads(q, w["q_norm"], dims.qk_norm_eps), pos, dims.rope_freq_dim, dims.rope_theta)
    kn = ob.rope_3d(ob.rms_norm_heads(k, w["k_norm"], dims.qk_norm_eps), pos, dims.rope_freq_dim, dims.rope_theta)
    o = ob.attention_doc_masked(qn, kn, v, ob.doc_ids(tags), 1.0 / np.sqrt(hd)).reshape(S, W)
    _, _, gate1 = ob.modulation(table, tags, tidx, 0)
    attn_proj = lin(o, w["w_out"])
    x_mid = x + gate1 * attn_proj
    b = ob.adaln(x_mid, table, tags, tidx, 1, dims.norm_eps)
    gu = lin(b, w["w_gate_up"])
    h = ob.silu(gu[:, :F]) * gu[:, F:]
    _, _, gate2 = ob.modulation(table, tags, tidx, 1)
    ffn_out = lin(h, w["w_down"])
    out = x_mid + gate2 * ffn_out
    if not taps:
        return out
    return out, dict(adaln1=round_bf16(a), attn_o=round_bf16(o), adaln2=round_bf16(b), ffn_h=round_bf16(h),
                     attn_proj=attn_proj, ffn_out=ffn_out)
