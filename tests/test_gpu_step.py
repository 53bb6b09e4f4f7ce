"""Parity of the denoising-step pieces (unmerged LoRA linear layer, Euler
update) against the fp64 oracle (GPU)."""
import numpy as np
import pytest
import torch

from helpers import REL_L2_F32, assert_close, gpu_available, rel_l2, to_np64
from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth
from oracle import step as ostep

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def bf16_pair(a):
    t = synth.Tensor(synth.round_to_bf16_bits(np.asarray(a, np.float32)), "bf16")
    return dv.to_device(t), t.values()


@pytest.mark.parametrize("M,N,K", [(300, 512, 512), (257, 768, 1024)])
@pytest.mark.parametrize("scale", [1.0, 0.5])
def test_linear_lora_bf16(M, N, K, scale):
    print(f"linear_lora bf16 M={M} N={N} K={K} scale={scale}", flush=True)
    r = 256
    rng = np.random.default_rng(M + N)
    a, av = bf16_pair(rng.standard_normal((M, K)))
    w, wv = bf16_pair(rng.standard_normal((N, K)) * 0.02)
    la, lav = bf16_pair(rng.standard_normal((r, K)) * 0.02)
    lb, lbv = bf16_pair(rng.standard_normal((N, r)) * 0.02)
    packed = m.lora_pack_weight(w, lb)
    out = m.linear_lora(a, la, packed, scale)
    torch.cuda.synchronize()
    ref = ostep.lora_linear(av, wv, lav, lbv, alpha=256.0, rank=256, scale=scale)
    assert_close(to_np64(out), ref, "linear_lora")


def test_lora_with_zero_b_is_the_plain_projection_bit_for_bit():
    M, N, K, r = 130, 256, 320, 256
    rng = np.random.default_rng(4)
    a, _ = bf16_pair(rng.standard_normal((M, K)))
    w, _ = bf16_pair(rng.standard_normal((N, K)) * 0.02)
    la, _ = bf16_pair(rng.standard_normal((r, K)))
    lb = torch.zeros(N, r, dtype=torch.bfloat16, device="cuda")
    got = m.linear_lora(a, la, m.lora_pack_weight(w, lb), 1.0)
    plain = m.linear(a, w)
    torch.cuda.synchronize()
    assert torch.equal(got, plain)


def test_linear_lora_f32():
    M, N, K, r = 70, 128, 64, 64
    rng = np.random.default_rng(5)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    la = rng.standard_normal((r, K)).astype(np.float32)
    lb = rng.standard_normal((N, r)).astype(np.float32)
    dev = lambda t: torch.from_numpy(t).cuda()  # noqa: E731
    out = m.linear_lora(dev(a), dev(la), m.lora_pack_weight(dev(w), dev(lb)), 0.25)
    torch.cuda.synchronize()
    ref = ostep.lora_linear(a, w, la, lb, alpha=64.0, rank=64, scale=0.25)
    assert rel_l2(to_np64(out), ref) <= REL_L2_F32


def test_linear_lora_full_qkv_shape_sampled_rows():
    print("linear_lora full QKV shape", flush=True)
    M, N, K, r = 32768, 21504, 5376, 256
    g = torch.Generator(device="cuda").manual_seed(1)
    a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    la = (torch.randn(r, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    lb = (torch.randn(N, r, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    out = m.linear_lora(a, la, m.lora_pack_weight(w, lb), 1.0)
    torch.cuda.synchronize()
    sel = np.array([0, 255, 256, 9999, 32767])
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ref = ostep.lora_linear(f64(a[sel]), f64(w), f64(la), f64(lb), alpha=256.0, rank=256)
    assert_close(f64(out[sel]), ref, "linear_lora full")


def test_euler_step_matches_and_keeps_pinned_rows():
    dims = synth.ModelDims(hidden=256, num_heads=2, ffn_dim=256, num_tvals=16, dtype="bf16")
    wl = synth.make_custom(dims, [("text", 9), ("audio", 11), ("video", 40, (2, 4, 5))], (2, 4, 5), 3, seed=6)
    L = wl.layout
    k = 4
    grid = (1.0 - np.arange(k) / k).astype(np.float32)
    v = np.arange(16)
    now, nxt = grid[v // k], grid[v % k]  # value v: the pair (g[v div 4], g[v mod 4]); the diagonal is r = t
    rng = np.random.default_rng(7)
    B, n, C = 2, len(L.video_indices), 96
    x = rng.standard_normal((B, n, C)).astype(np.float32)
    vel = rng.standard_normal((B, n, C)).astype(np.float32)
    cu = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()  # noqa: E731
    idx, tidx = cu(L.video_indices.astype(np.int32)), cu(L.timestep_indices.astype(np.int32))
    got = m.euler_step(cu(x), cu(vel), idx, tidx, cu(now), cu(nxt))
    torch.cuda.synchronize()
    rt = L.timestep_indices[L.video_indices]
    ref = ostep.euler_step(x, vel, np.broadcast_to(now[rt], (B, n)), np.broadcast_to(nxt[rt], (B, n)))
    g64 = got.cpu().numpy().astype(np.float64)
    assert np.abs(g64 - ref).max() <= 1e-6 * np.abs(ref).max()
    pinned = now[rt] == nxt[rt]
    assert pinned.any() and np.array_equal(got.cpu().numpy()[:, pinned], x[:, pinned])
    # in place
    xi = cu(x)
    m.euler_step(xi, cu(vel), idx, tidx, cu(now), cu(nxt), out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, got)
