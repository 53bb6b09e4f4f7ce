"""Full-size parity (GPU): the five named workloads in the launch configuration
bench.py times, against the fp64 oracle.

The tiny workload is compared on every element (test_gpu_block.py). The four
full-width workloads are compared on sampled rows whose oracle values were
written by tests/golden/make_golden.py (oracle only); properties that hold
at any size are checked bit-exactly on every row.
"""
import os

import numpy as np
import pytest
import torch

from helpers import assert_close, gpu_available, to_np64
from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    path = os.path.join(GOLDEN, f"{name}_seed0.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} missing (python tests/golden/make_golden.py {name})")
    return dict(np.load(path, allow_pickle=False))


@pytest.mark.parametrize("name", ["padless8k", "padded16k", "clip32k"])
def test_single_block_full_size(name):
    print(f"full-size block: {name}", flush=True)
    g = golden(name)
    wl = synth.make_workload(name, seed=0)
    assert wl.layout.seq_len == int(g["seq_len"]) and wl.layout.num_pad == int(g["num_pad"])
    cfg, lay, blocks, x = dv.upload(wl)
    rows = torch.from_numpy(g["rows"]).cuda()
    B, S, W = 1, lay.seq_len, cfg.num_heads * cfg.head_dim
    attn_o = torch.empty(B, S, W, dtype=torch.bfloat16, device="cuda")
    out = m.block_forward(cfg, lay, blocks, x, flags=m.VALIDATE, taps={"attn_o": attn_o})
    torch.cuda.synchronize()
    assert_close(to_np64(out[0, rows]), g["out"].astype(np.float64), f"{name} out")
    assert_close(to_np64(attn_o[0, rows]), g["attn_o"].astype(np.float64), f"{name} attn_o")
    # any size: padding rows leave the block bit-unchanged; everything is finite
    pad = torch.from_numpy(wl.layout.token_tags == -1).cuda()
    assert torch.equal(out[:, pad], x[:, pad])
    assert torch.isfinite(out.float()).all()


def test_chain_of_four_full_size():
    print("full-size chain of 4 blocks", flush=True)
    g = golden("chain4x24k")
    wl = synth.make_workload("chain4x24k", seed=0)
    assert wl.layout.seq_len == int(g["seq_len"]) and wl.layout.num_pad == int(g["num_pad"])
    cfg, lay, blocks, x = dv.upload(wl)
    del wl.blocks[:]
    rows = torch.from_numpy(g["rows"]).cuda()
    out = m.block_forward(cfg, lay, blocks, x, flags=m.VALIDATE)
    one = m.block_forward(cfg, lay, blocks[:1], x)
    torch.cuda.synchronize()
    assert_close(to_np64(out[0, rows]), g["out"].astype(np.float64), "chain out")
    assert_close(to_np64(one[0, rows]), g["block1_out"].astype(np.float64), "chain block 1")
    pad = torch.from_numpy(wl.layout.token_tags == -1).cuda()
    assert torch.equal(out[:, pad], x[:, pad])


def test_padless_flag_bit_exact_full_size():
    # the mask-free promise changes nothing when no padding row is present
    print("full-size padless flag", flush=True)
    wl = synth.make_workload("padless8k", seed=0)
    cfg, lay, blocks, x = dv.upload(wl)
    a = m.block_forward(cfg, lay, blocks, x)
    b = m.block_forward(cfg, lay, blocks, x, flags=m.ASSUME_PADLESS | m.VALIDATE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_pad_content_independence_full_size():
    # re-randomised padding rows (same count) leave every real row bit-identical
    print("full-size pad independence", flush=True)
    wl = synth.make_workload("padded16k", seed=0)
    cfg, lay, blocks, x = dv.upload(wl)
    pad = torch.from_numpy(wl.layout.token_tags == -1).cuda()
    a = m.block_forward(cfg, lay, blocks, x)
    x2 = x.clone()
    x2[:, pad] = (torch.randn(1, int(pad.sum()), cfg.hidden, device="cuda") * 3).to(x.dtype)
    b = m.block_forward(cfg, lay, blocks, x2)
    torch.cuda.synchronize()
    assert torch.equal(a[:, ~pad], b[:, ~pad])
