"""Parity of the model edges (input projections with the scatter into the
packed sequence, norm_out and the output heads with the gather) against the
fp64 oracle (GPU).

Called through the C ABI: small layouts with ragged row counts (not multiples
of the 64-row tiles), both activation types, and the full clip-scale layout
(30208 video, 1536 audio, 1024 text rows, hidden 5376). Text rows must be
copied bit-exactly and padding rows must be exactly zero.
"""
import numpy as np
import pytest
import torch

from helpers import REL_L2_F32, assert_close, gpu_available, max_abs, rel_l2, to_np64
from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth
from oracle import edges as oe

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def small(dtype, pads=13, batch=2, seed=0):
    dims = synth.ModelDims(hidden=512, num_heads=4, ffn_dim=768, num_tvals=8, dtype=dtype)
    segs = [("text", 37), ("cond", 20, (1, 4, 5)), ("audio", 29), ("video", 105, (3, 5, 7))]
    wl = synth.make_custom(dims, segs, (3, 5, 7), pads, seed=seed, batch=batch)
    return dims, wl.layout, synth.make_edges(dims, wl.layout, batch=batch, seed=seed + 1)


def assert_f32(got, ref, name):
    assert np.all(np.isfinite(got)), name
    r, mx = rel_l2(got, ref), max_abs(got, ref)
    assert r <= REL_L2_F32 and mx <= 1e-4 * max(1.0, float(np.abs(ref).max())), f"{name}: rel {r:.3e} max {mx:.3e}"


def run_embed(dims, L, e, batch, flags=0):
    cfg = dv.config_for(dims)
    lay = m.DeviceLayout(batch, L.token_tags, L.timestep_indices, L.position_ids, L.video_indices, L.audio_indices,
                         L.text_indices)
    x = m.embed_inputs(cfg, lay, dv.edges_for(e), dv.f32(e.video), dv.f32(e.audio), dv.to_device(e.text),
                       flags=flags)
    torch.cuda.synchronize()
    return cfg, lay, x


def check_embed(dims, L, e, x_dev):
    ref = oe.embed_inputs(e.video, e.audio, e.text.values(), L, e.w_in, e.b_in, e.w_ain, e.b_ain, dims.hidden)
    got = to_np64(x_dev)
    vi = np.concatenate([L.video_indices, L.audio_indices])
    if dims.dtype == "bf16":
        assert_close(got[:, vi], ref[:, vi], "embedded rows")
        # one bf16 rounding of an fp32 result
        assert np.all(np.abs(got[:, vi] - ref[:, vi]) <= 2.0 ** -8 * np.abs(ref[:, vi]) + 1e-5)
    else:
        assert_f32(got[:, vi], ref[:, vi], "embedded rows")
    # text rows are copies, padding rows zero: bit-exact
    assert np.array_equal(got[:, L.text_indices], e.text.values())
    pad = L.token_tags == -1
    assert np.all(got[:, pad] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_embed_inputs_small(dtype):
    dims, L, e = small(dtype)
    _, _, x = run_embed(dims, L, e, 2, flags=m.VALIDATE)
    check_embed(dims, L, e, x)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_output_heads_small(dtype):
    dims, L, e = small(dtype, pads=3, seed=4)
    cfg, lay, x = run_embed(dims, L, e, 2)
    v, a = m.output_heads(cfg, lay, dv.edges_for(e), x, flags=m.VALIDATE)
    torch.cuda.synchronize()
    rv, ra = oe.output_heads(to_np64(x), L, e.gamma, e.beta, e.final_norm_eps, e.w_out, e.b_out, e.w_aout, e.b_aout)
    assert_f32(to_np64(v), rv, "video head")
    assert_f32(to_np64(a), ra, "audio head")


def test_output_heads_rows_with_large_mean():
    # LayerNorm statistics stay exact for rows far from zero mean (the kernel
    # accumulates x - x_0 and its square)
    dims, L, e = small("f32", pads=3, seed=6, batch=1)
    cfg, lay, x = run_embed(dims, L, e, 1)
    x = x + 300.0
    v, a = m.output_heads(cfg, lay, dv.edges_for(e), x)
    torch.cuda.synchronize()
    rv, ra = oe.output_heads(to_np64(x), L, e.gamma, e.beta, e.final_norm_eps, e.w_out, e.b_out, e.w_aout, e.b_aout)
    assert_f32(to_np64(v), rv, "video head")
    assert_f32(to_np64(a), ra, "audio head")


def test_embed_inputs_reports_invalid_layouts():
    dims, L, e = small("bf16", batch=1)
    bad = L.video_indices.copy()
    bad[3] = bad[4]  # a row addressed twice, another not at all
    lay = m.DeviceLayout(1, L.token_tags, L.timestep_indices, L.position_ids, bad, L.audio_indices, L.text_indices)
    cfg = dv.config_for(dims)
    with pytest.raises(m.Minih3Error) as ei:
        m.embed_inputs(cfg, lay, dv.edges_for(e), dv.f32(e.video), dv.f32(e.audio), dv.to_device(e.text),
                       flags=m.VALIDATE)
    assert ei.value.status == m.E_LAYOUT_INDEX


@pytest.mark.parametrize("segs,grid", [
    ([("text", 21), ("video", 70, (2, 5, 7))], (2, 5, 7)),  # no audio rows
    ([("text", 9), ("audio", 45)], (4, 1, 1)),              # no video rows: the narrower head alone
    ([("text", 30)], (1, 1, 1)),                            # neither head has rows
])
def test_edges_with_a_modality_absent(segs, grid):
    print(f"edges without a modality {[sg[:2] for sg in segs]}", flush=True)
    dims = synth.ModelDims(hidden=512, num_heads=4, ffn_dim=768, num_tvals=8, dtype="bf16")
    L = synth.make_custom(dims, segs, grid, 5, seed=9).layout
    e = synth.make_edges(dims, L, seed=10)
    cfg, lay, x = run_embed(dims, L, e, 1, flags=m.VALIDATE)
    check_embed(dims, L, e, x)
    v, a = m.output_heads(cfg, lay, dv.edges_for(e), x, flags=m.VALIDATE)
    torch.cuda.synchronize()
    rv, ra = oe.output_heads(to_np64(x), L, e.gamma, e.beta, e.final_norm_eps, e.w_out, e.b_out, e.w_aout, e.b_aout)
    assert tuple(v.shape) == rv.shape and tuple(a.shape) == ra.shape
    if rv.size:
        assert_f32(to_np64(v), rv, "video head")
    if ra.size:
        assert_f32(to_np64(a), ra, "audio head")


def test_edges_full_clip_scale():
    print("edges full clip scale", flush=True)
    wl = synth.make_workload("clip32k", with_weights=False)
    dims, L = wl.dims, wl.layout
    e = synth.make_edges(dims, L, seed=3)
    cfg, lay, x = run_embed(dims, L, e, 1)
    check_embed(dims, L, e, x)
    v, a = m.output_heads(cfg, lay, dv.edges_for(e), x)
    torch.cuda.synchronize()
    rv, ra = oe.output_heads(to_np64(x), L, e.gamma, e.beta, e.final_norm_eps, e.w_out, e.b_out, e.w_aout, e.b_aout)
    assert v.shape == (1, 30208, 96) and a.shape == (1, 1536, 32)
    assert_f32(to_np64(v), rv, "video head")
    assert_f32(to_np64(a), ra, "audio head")
