"""A seeded sweep of small block shapes against the fp64 oracle (GPU).

Each case draws its model widths (hidden 256..1024, 2..8 heads, FFN
128..1024, 0..21 rotary frequencies per axis, 1..8 timestep values), its
layout (segment sizes, video grids, padding rows) and its batch size from a
fixed seed, so that the block runs at widths and sequence lengths none of the
hand-picked cases uses: ragged GEMM, attention and RoPE tails, batch items
that share a 256-row tile, tables of one timestep value. Every tap and the
output are held to the graded bar (fp32 cases also to the fp32 bar), the
increments of both gated adds to relative L2 1e-2, and the integer layout taps
bit for bit (check_block of test_gpu_block).
"""
import numpy as np
import pytest

from helpers import MAX_ABS_F32, REL_L2_F32, gpu_available
from joint_video_audio_amd import synth
from test_gpu_block import check_block

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _cases(n, seed, dtype):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hidden = int(rng.choice([256, 512, 768, 1024]))
        heads = int(rng.choice([2, 4, 6, 8]))
        ffn = int(rng.choice([128, 256, 384, 640, 1024]))
        fd = int(rng.choice([0, 4, 8, 16, 21]))
        tv = int(rng.choice([1, 3, 8]))
        batch = int(rng.choice([1, 2, 3]))
        t, h, w = (int(v) for v in rng.integers(1, 9, size=3))
        segs = [("video", t * h * w, (t, h, w))]
        if rng.random() < 0.8:
            segs.append(("text", int(rng.integers(1, 200))))
        if rng.random() < 0.7:
            segs.append(("audio", int(rng.integers(1, 120))))
        if rng.random() < 0.5:
            ch, cw = (int(v) for v in rng.integers(1, 5, size=2))
            segs.append(("cond", ch * cw, (1, ch, cw)))
        pads = int(rng.choice([0, 1, 17, 64, 130]))
        out.append(pytest.param(dict(hidden=hidden, num_heads=heads, ffn_dim=ffn, rope_freq_dim=fd, num_tvals=tv,
                                     dtype=dtype), segs, (t, h, w), pads, batch, seed * 100 + i,
                                id=f"{dtype}-{i}-D{hidden}-H{heads}-F{ffn}-fd{fd}-B{batch}-p{pads}"))
    return out


@pytest.mark.parametrize("dims,segs,grid,pads,batch,seed", _cases(10, 11, "bf16") + _cases(3, 12, "f32"))
def test_block_shape_sweep(dims, segs, grid, pads, batch, seed):
    print(f"sweep {dims} segs={[s[:2] for s in segs]} pads={pads} batch={batch}", flush=True)
    wl = synth.make_custom(synth.ModelDims(**dims), segs, grid, pads, seed=seed, batch=batch)
    if dims["dtype"] == "f32":
        check_block(wl, rel=REL_L2_F32, mabs=MAX_ABS_F32)
    else:
        check_block(wl)
