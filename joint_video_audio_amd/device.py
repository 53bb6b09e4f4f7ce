"""Upload a synthetic workload to the device in the library's formats."""
from __future__ import annotations

import numpy as np
import torch

from . import minih3 as m
from .synth import NUM_TAGS, TAG_AUDIO, TAG_TEXT, TAG_VIDEO, Tensor, Workload


def config_for(dims) -> m.Config:
    return m.Config(dims.hidden, dims.num_heads, dims.head_dim, dims.ffn_dim, dims.rope_freq_dim,
                    float(dims.rope_theta), float(dims.norm_eps), float(dims.qk_norm_eps), NUM_TAGS,
                    dims.num_tvals, TAG_TEXT, TAG_VIDEO, TAG_AUDIO, m.BF16 if dims.dtype == "bf16" else m.F32)


def to_device(t: Tensor, device="cuda") -> torch.Tensor:
    """Exact device copy of a stored host tensor (bf16 bit patterns or fp32)."""
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)


def f32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def layout_for(wl: Workload, device="cuda", batch=None) -> m.DeviceLayout:
    L = wl.layout
    return m.DeviceLayout(wl.batch if batch is None else batch, L.token_tags, L.timestep_indices, L.position_ids,
                          L.video_indices, L.audio_indices, L.text_indices, device=device)


def block_for(bw, device="cuda") -> m.DeviceBlock:
    return m.DeviceBlock(to_device(bw.w_qkv, device), to_device(bw.w_out, device), to_device(bw.w_gate_up, device),
                         to_device(bw.w_down, device), f32(bw.q_norm, device), f32(bw.k_norm, device),
                         f32(bw.adaln_table, device))


def upload(wl: Workload, device="cuda"):
    """(config, layout, [blocks], x) on the device."""
    return config_for(wl.dims), layout_for(wl, device), [block_for(b, device) for b in wl.blocks], \
        to_device(wl.x, device)


def time_config_for(cond, max_period: float = 1.0e4) -> m.TimeConfig:
    return m.TimeConfig(cond.freq_dim, cond.hidden_dim, cond.embed_dim, float(max_period))


def time_mlp_for(te, device="cuda") -> m.DeviceTimeMLP:
    return m.DeviceTimeMLP(f32(te.w1, device), f32(te.b1, device), f32(te.w2, device), f32(te.b2, device))


def edges_for(e, device="cuda") -> m.DeviceEdges:
    """Device copies of synthetic edge weights (synth.Edges)."""
    return m.DeviceEdges(e.w_in.shape[1], e.w_ain.shape[1], e.final_norm_eps,
                         **{n: f32(getattr(e, a), device) for n, a in (
                             ("w_in", "w_in"), ("b_in", "b_in"), ("w_audio_in", "w_ain"), ("b_audio_in", "b_ain"),
                             ("norm_w", "gamma"), ("norm_b", "beta"), ("w_out", "w_out"), ("b_out", "b_out"),
                             ("w_audio_out", "w_aout"), ("b_audio_out", "b_aout"))})
