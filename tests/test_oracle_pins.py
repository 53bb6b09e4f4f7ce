"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form, an
invariant the MiniMaxH3Transformer3DModel page states, or brute force on a
tiny input, so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import block as ob
from oracle import layout as ol
from oracle import weights_f64
from joint_video_audio_amd import synth

RTOL = 1e-12


def small_dims(**kw):
    d = dict(hidden=256, num_heads=2, head_dim=128, ffn_dim=384, num_tvals=4, dtype="f32")
    d.update(kw)
    return synth.ModelDims(**d)


def small_workload(pads=5, seed=0, batch=1, dims=None):
    dims = dims or small_dims()
    segs = [("text", 7), ("cond", 6, (1, 2, 3)), ("audio", 5), ("video", 24, (2, 3, 4))]
    return synth.make_custom(dims, segs, (2, 3, 4), pads, seed=seed, batch=batch)


def close(a, b, tol=RTOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, float(np.abs(a - b).max())


# ---------------------------------------------------------------- AdaLN

def test_layer_norm_matches_torch_and_closed_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((17, 96)) * 3 + 0.7
    y = ob.layer_norm(x, 1e-5)
    ref = F.layer_norm(torch.from_numpy(x), (96,), eps=1e-5).numpy()
    close(y, ref)
    var = x.var(axis=1)
    close(y.mean(axis=1), np.zeros(17))
    close(y.var(axis=1), var / (var + 1e-5))


def test_modulation_gathers_tag_and_timestep():
    # table[m, k, c, :] = 100 m + 10 k + c identifies its entry.
    n_tags, n_tv, D = 3, 4, 8
    m, k, c = np.meshgrid(np.arange(n_tags), np.arange(n_tv), np.arange(6), indexing="ij")
    table = (100 * m + 10 * k + c)[..., None].repeat(D, -1).astype(np.float64)
    tags = np.array([0, 2, -1, 1, 2])
    tidx = np.array([3, 1, 2, 0, 2])
    for which in (0, 1):
        shift, scale, gate = ob.modulation(table, tags, tidx, which)
        for i, (t, kk) in enumerate(zip(tags, tidx)):
            want = [0, 0, 0] if t == -1 else [100 * t + 10 * kk + 3 * which + c for c in range(3)]
            assert shift[i, 0] == want[0] and scale[i, 0] == want[1] and gate[i, 0] == want[2]


def test_adaln_is_affine_layer_norm_per_group():
    # For rows sharing (tag, tidx), AdaLN equals torch's affine layer_norm
    # with weight 1 + scale and bias shift.
    rng = np.random.default_rng(2)
    D = 64
    table = rng.standard_normal((3, 2, 6, D)) * 0.3
    tags = np.array([1] * 6 + [-1] * 2)
    tidx = np.array([1] * 6 + [0] * 2)
    x = rng.standard_normal((8, D))
    for which in (0, 1):
        y = ob.adaln(x, table, tags, tidx, which, 1e-5)
        w = torch.from_numpy(1 + table[1, 1, 3 * which + 1])
        b = torch.from_numpy(table[1, 1, 3 * which + 0])
        ref = F.layer_norm(torch.from_numpy(x[:6]), (D,), w, b, eps=1e-5).numpy()
        close(y[:6], ref)
        close(y[6:], F.layer_norm(torch.from_numpy(x[6:]), (D,), eps=1e-5).numpy())


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_matches_torch_and_unit_rms():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 3, 128)) * 2.5
    g = 1 + 0.1 * rng.standard_normal(128)
    ref = F.rms_norm(torch.from_numpy(q), (128,), torch.from_numpy(g), eps=1e-5).numpy()
    close(ob.rms_norm_heads(q, g, 1e-5), ref)
    y = ob.rms_norm_heads(q, np.ones(128), 1e-5)
    ms = (q ** 2).mean(-1)
    close(np.sqrt((y ** 2).mean(-1)), np.sqrt(ms / (ms + 1e-5)))


# ---------------------------------------------------------------- RoPE

def complex_rope_reference(q, pos, fd, theta):
    """Rotary embedding as complex multiplication (torch.polar), with the
    inv_freq written in the common 1 / theta^(arange(0, 2fd, 2) / 2fd) form."""
    q = torch.from_numpy(q)
    out = q.clone()
    inv = 1.0 / (theta ** (torch.arange(0, 2 * fd, 2, dtype=torch.float64) / (2 * fd)))
    for a in range(3):
        blk = q[..., 2 * fd * a: 2 * fd * (a + 1)].reshape(*q.shape[:-1], fd, 2).contiguous()
        zc = torch.view_as_complex(blk)
        ang = torch.outer(torch.from_numpy(pos[:, a]).double(), inv)[:, None, :]
        rot = zc * torch.polar(torch.ones_like(ang), ang)
        out[..., 2 * fd * a: 2 * fd * (a + 1)] = torch.view_as_real(rot).reshape(*q.shape[:-1], 2 * fd)
    return out.numpy()


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((9, 2, 128))
    pos = rng.integers(0, 2048, size=(9, 3))
    close(ob.rope_3d(q, pos, 16, 1e4), complex_rope_reference(q, pos, 16, 1e4), 1e-10)


def test_rope_identity_norms_passthrough():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 2, 128))
    close(ob.rope_3d(q, np.zeros((6, 3), np.int64), 16, 1e4), q)      # position 0 = identity
    pos = rng.integers(0, 1000, size=(6, 3))
    y = ob.rope_3d(q, pos, 16, 1e4)
    assert np.array_equal(y[..., 96:], q[..., 96:])                  # 96 of 128 rotated
    n0 = q[..., :96:2] ** 2 + q[..., 1:96:2] ** 2
    n1 = y[..., :96:2] ** 2 + y[..., 1:96:2] ** 2
    close(n1, n0)                                                     # each pair keeps its norm


def test_rope_scores_depend_on_relative_position():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 1, 128))
    k = rng.standard_normal((4, 1, 128))
    pq = rng.integers(0, 500, size=(4, 3))
    pk = rng.integers(0, 500, size=(4, 3))
    d = np.array([[37, -11, 250]])
    s0 = np.einsum("ihd,jhd->ij", ob.rope_3d(q, pq, 16, 1e4), ob.rope_3d(k, pk, 16, 1e4))
    s1 = np.einsum("ihd,jhd->ij", ob.rope_3d(q, pq + d, 16, 1e4), ob.rope_3d(k, pk + d, 16, 1e4))
    close(s0, s1, 1e-10)


def test_rope_direction_and_frequency():
    # unit vector on pair j of axis a at position p turns by p * theta^(-j/16),
    # counter-clockwise: (1, 0) -> (cos, sin)
    for a, j, p in [(0, 0, 1), (1, 5, 7), (2, 15, 1000)]:
        q = np.zeros((1, 1, 128))
        q[0, 0, 32 * a + 2 * j] = 1.0
        pos = np.zeros((1, 3), np.int64)
        pos[0, a] = p
        y = ob.rope_3d(q, pos, 16, 1e4)[0, 0]
        phi = p * 1e4 ** (-j / 16)
        assert abs(y[32 * a + 2 * j] - math.cos(phi)) < 1e-12
        assert abs(y[32 * a + 2 * j + 1] - math.sin(phi)) < 1e-12


# ---------------------------------------------------------------- attention

def brute_attention(q, k, v, doc, scale):
    S, H, hd = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(S):
            ks = [j for j in range(S) if doc[j] == doc[i]]
            scores = [sum(q[i, h, d] * k[j, h, d] for d in range(hd)) * scale for j in ks]
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            tot = sum(e)
            for d in range(hd):
                out[i, h, d] = sum(e[n] * v[ks[n], h, d] for n in range(len(ks))) / tot
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(7)
    S, H, hd = 11, 2, 8
    q, k, v = (rng.standard_normal((S, H, hd)) for _ in range(3))
    doc = np.array([0, 0, 1, 0, 0, 1, 0, 0, 0, 1, 0])
    close(ob.attention_doc_masked(q, k, v, doc, 0.7), brute_attention(q, k, v, doc, 0.7))


def test_attention_padless_matches_sdpa():
    rng = np.random.default_rng(8)
    S, H, hd = 70, 3, 128
    q, k, v = (rng.standard_normal((S, H, hd)) for _ in range(3))
    out = ob.attention_doc_masked(q, k, v, np.zeros(S, np.int64), 1 / math.sqrt(hd))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v))[0].permute(1, 0, 2).numpy()
    close(out, ref)


def test_attention_padded_equals_truncated_and_special_cases():
    rng = np.random.default_rng(9)
    S, H, hd, P = 40, 2, 16, 6
    q, k, v = (rng.standard_normal((S, H, hd)) for _ in range(3))
    doc = np.r_[np.zeros(S - P, np.int64), np.ones(P, np.int64)]
    full = ob.attention_doc_masked(q, k, v, doc, 0.3)
    trunc = ob.attention_doc_masked(q[:S - P], k[:S - P], v[:S - P], doc[:S - P], 0.3)
    tail = ob.attention_doc_masked(q[S - P:], k[S - P:], v[S - P:], doc[S - P:] * 0, 0.3)
    close(full[:S - P], trunc)
    close(full[S - P:], tail)
    # a one-row padding document attends only to itself
    doc1 = np.zeros(S, np.int64)
    doc1[13] = 1
    close(ob.attention_doc_masked(q, k, v, doc1, 0.3)[13], v[13])
    # identical keys: uniform weights, the output is the mean of V
    kk = np.repeat(k[:1], S, axis=0)
    close(ob.attention_doc_masked(q, kk, v, np.zeros(S, np.int64), 0.3), np.repeat(v.mean(0, keepdims=True), S, 0))


def test_attention_query_subset():
    rng = np.random.default_rng(10)
    S, H, hd = 33, 2, 16
    q, k, v = (rng.standard_normal((S, H, hd)) for _ in range(3))
    doc = (rng.random(S) < 0.2).astype(np.int64)
    rows = np.array([0, 5, 32, 7])
    close(ob.attention_doc_masked(q, k, v, doc, 0.25, rows=rows),
          ob.attention_doc_masked(q, k, v, doc, 0.25)[rows])


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(11)
    b = rng.standard_normal((5, 32))
    w = rng.standard_normal((2 * 48, 32))
    g = torch.from_numpy(b @ w[:48].T)
    u = torch.from_numpy(b @ w[48:].T)
    close(ob.swiglu(b, w, 48), (F.silu(g) * u).numpy())
    w2 = w.copy()
    w2[48:] = 0
    assert np.all(ob.swiglu(b, w2, 48) == 0)


# ---------------------------------------------------------------- block

def library_block(x, layout, w, dims):
    """The block built from torch library routines (fp64 CPU)."""
    S, D = x.shape
    H, hd, Fd = dims.num_heads, dims.head_dim, dims.ffn_dim
    W = H * hd
    tags = torch.from_numpy(layout.token_tags.astype(np.int64))
    tidx = torch.from_numpy(layout.timestep_indices.astype(np.int64))
    table = torch.from_numpy(w["adaln_table"])
    real = tags >= 0
    mod = torch.zeros(S, 6, D, dtype=torch.float64)
    mod[real] = table[tags[real], tidx[real]]
    xt = torch.from_numpy(x)
    a = F.layer_norm(xt, (D,), eps=dims.norm_eps) * (1 + mod[:, 1]) + mod[:, 0]
    qkv = F.linear(a, torch.from_numpy(w["w_qkv"]))
    q, k, v = qkv.split(W, dim=-1)
    q = F.rms_norm(q.reshape(S, H, hd), (hd,), torch.from_numpy(w["q_norm"]), eps=dims.qk_norm_eps)
    k = F.rms_norm(k.reshape(S, H, hd), (hd,), torch.from_numpy(w["k_norm"]), eps=dims.qk_norm_eps)
    pos = layout.position_ids.astype(np.int64)
    q = torch.from_numpy(complex_rope_reference(q.numpy(), pos, dims.rope_freq_dim, dims.rope_theta))
    k = torch.from_numpy(complex_rope_reference(k.numpy(), pos, dims.rope_freq_dim, dims.rope_theta))
    pad = ~real
    mask = pad[:, None] == pad[None, :]
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                       v.reshape(S, H, hd).permute(1, 0, 2)[None], attn_mask=mask)
    o = o[0].permute(1, 0, 2).reshape(S, W)
    x_mid = xt + mod[:, 2] * F.linear(o, torch.from_numpy(w["w_out"]))
    b = F.layer_norm(x_mid, (D,), eps=dims.norm_eps) * (1 + mod[:, 4]) + mod[:, 3]
    gu = F.linear(b, torch.from_numpy(w["w_gate_up"]))
    h = F.silu(gu[:, :Fd]) * gu[:, Fd:]
    return (x_mid + mod[:, 5] * F.linear(h, torch.from_numpy(w["w_down"]))).numpy()


def test_block_matches_library_block():
    wl = small_workload(pads=5)
    w = weights_f64(wl.blocks[0])
    x = wl.x.values()[0]
    close(ob.block_forward(x, wl.layout, w, wl.dims), library_block(x, wl.layout, w, wl.dims), 1e-10)


def test_block_gate_zero_is_identity_and_rows_subset():
    wl = small_workload(pads=3)
    w = weights_f64(wl.blocks[0])
    x = wl.x.values()[0]
    w0 = dict(w)
    w0["adaln_table"] = w["adaln_table"].copy()
    w0["adaln_table"][:, :, 2] = 0
    w0["adaln_table"][:, :, 5] = 0
    assert np.array_equal(ob.block_forward(x, wl.layout, w0, wl.dims), x)
    full = ob.block_forward(x, wl.layout, w, wl.dims)
    rows = np.array([3, 0, 44, 40, 20])
    close(ob.block_forward(x, wl.layout, w, wl.dims, rows=rows), full[rows])
    # padding rows leave the block unchanged
    pad = wl.layout.token_tags == -1
    assert np.array_equal(full[pad], x[pad])


def test_block_row_permutation_equivariance():
    wl = small_workload(pads=4)
    w = weights_f64(wl.blocks[0])
    x = wl.x.values()[0]
    perm = np.random.default_rng(12).permutation(wl.layout.seq_len)
    lay_p = synth.permute_rows(wl.layout, perm)
    close(ob.block_forward(x[perm], lay_p, w, wl.dims), ob.block_forward(x, wl.layout, w, wl.dims)[perm], 1e-10)


def test_block_padding_rows_never_influence_real_rows():
    wl = small_workload(pads=4)
    w = weights_f64(wl.blocks[0])
    x = wl.x.values()[0]
    real = wl.layout.token_tags != -1
    base = ob.block_forward(x, wl.layout, w, wl.dims)
    # re-randomised pad contents
    x2 = x.copy()
    x2[~real] = np.random.default_rng(13).standard_normal((int((~real).sum()), x.shape[1])) * 5
    close(ob.block_forward(x2, wl.layout, w, wl.dims)[real], base[real], 0)
    # a different pad count (pads dropped entirely): real rows unchanged
    lay = wl.layout
    keep = np.flatnonzero(real)
    lay_t = synth.Layout(lay.token_tags[keep], lay.timestep_indices[keep], lay.position_ids[keep],
                         lay.video_indices, lay.audio_indices, lay.text_indices)
    close(ob.block_forward(x[keep], lay_t, w, wl.dims), base[real], 1e-10)


def test_block_batch_replication_and_identical_rows():
    wl = small_workload(pads=2, batch=2)
    w = weights_f64(wl.blocks[0])
    xb = wl.x.values()
    out = ob.block_forward_batched(xb, wl.layout, w, wl.dims)
    close(out[1], ob.block_forward(xb[1], wl.layout, w, wl.dims), 0)
    # identical (x, tag, tidx, pos) rows give identical outputs
    x = xb[0].copy()
    lay = wl.layout
    tags = lay.token_tags.copy(); tidx = lay.timestep_indices.copy(); pos = lay.position_ids.copy()
    i, j = 20, 30                                      # two video rows
    x[j] = x[i]; tidx[j] = tidx[i]; pos[j] = pos[i]
    lay2 = synth.Layout(tags, tidx, pos, lay.video_indices, lay.audio_indices, lay.text_indices)
    y = ob.block_forward(x, lay2, w, wl.dims)
    close(y[j], y[i], 1e-13)


def test_chain_is_sequential_blocks():
    dims = small_dims()
    segs = [("text", 5), ("audio", 4), ("video", 12, (1, 3, 4))]
    wl = synth.make_custom(dims, segs, (1, 3, 4), 3, seed=3, num_blocks=3)
    ws = [weights_f64(b) for b in wl.blocks]
    x = wl.x.values()[0]
    y = x
    for w in ws:
        y = ob.block_forward(y, wl.layout, w, dims)
    assert np.array_equal(ob.chain_forward(x, wl.layout, ws, dims), y)


# ---------------------------------------------------------------- layout

def _describe(lay, n_tv=8, padless=False):
    return ol.describe(lay.token_tags, lay.timestep_indices, lay.video_indices, lay.audio_indices,
                       lay.text_indices, 3, n_tv, 1, 2, 0, padless)


def test_layout_describe_valid_and_errors():
    wl = synth.make_workload("tiny", with_weights=False)
    lay = wl.layout
    d = _describe(lay)
    assert d["status"] == 0 and d["num_pad"] == 16
    tags, tidx = lay.token_tags, lay.timestep_indices
    assert d["table_row"][0] == tags[0] * 8 + tidx[0] and d["table_row"][-1] == -1
    assert d["tile_flags"].tolist() == [1, 1, 1, 1, 3]    # 320 rows, pads in the last 16
    assert _describe(lay, padless=True)["status"] == ol.E_NEEDS_MASK

    def mutate(**kw):
        L = synth.Layout(**{**lay.__dict__, **{k: np.array(v, np.int32) for k, v in kw.items()}})
        return _describe(L)["status"]

    t = tags.copy(); t[5] = 3
    assert mutate(token_tags=t) == ol.E_TAG
    k = tidx.copy(); k[7] = 8
    assert mutate(timestep_indices=k) == ol.E_TVAL
    k = tidx.copy(); k[-1] = 99                         # ignored on padding rows
    assert mutate(timestep_indices=k) == 0
    v = lay.video_indices.copy(); v[0] = v[1]            # duplicate
    assert mutate(video_indices=v) == ol.E_INDEX
    v = lay.video_indices.copy(); v[0] = 400             # out of range
    assert mutate(video_indices=v) == ol.E_INDEX
    v = lay.video_indices.copy(); v[0] = 0               # a text row
    assert mutate(video_indices=v) == ol.E_INDEX
    v = lay.video_indices.copy(); v[0] = 310             # a padding row
    assert mutate(video_indices=v) == ol.E_PAD
    assert mutate(video_indices=lay.video_indices[1:]) == ol.E_PAD   # uncovered real row
