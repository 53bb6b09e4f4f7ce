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


@pytest.mark.parametrize("M,N,K", [(300, 512, 512), (257, 768, 1024), (65, 256, 64)])
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


def test_euler_step_two_schedules():
    # video and audio latents follow their own sigma schedules (shift 12 and
    # shift 3) in one call: the audio rows carry their own timestep values, so
    # one pair of per-value sigma tables serves both
    dims = synth.ModelDims(hidden=256, num_heads=2, ffn_dim=256, num_tvals=16, dtype="bf16")
    wl = synth.make_custom(dims, [("text", 5), ("audio", 21), ("video", 48, (2, 4, 6))], (2, 4, 6), 0, seed=11)
    L = wl.layout
    tidx = L.timestep_indices.copy()
    step = 3  # grid position of this step (of 8)
    tidx[L.video_indices] = step
    tidx[L.audio_indices] = 8 + step
    grid = 1.0 - np.arange(9) / 8.0
    now = np.concatenate([ostep.shift_sigmas(grid[:8], 12.0), ostep.shift_sigmas(grid[:8], 3.0)]).astype(np.float32)
    nxt = np.concatenate([ostep.shift_sigmas(grid[1:], 12.0), ostep.shift_sigmas(grid[1:], 3.0)]).astype(np.float32)
    rng = np.random.default_rng(12)
    cu = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()  # noqa: E731
    tid = cu(tidx.astype(np.int32))
    for idx, C, shift in ((L.video_indices, 96, 12.0), (L.audio_indices, 32, 3.0)):
        x = rng.standard_normal((1, len(idx), C)).astype(np.float32)
        v = rng.standard_normal((1, len(idx), C)).astype(np.float32)
        got = m.euler_step(cu(x), cu(v), cu(idx.astype(np.int32)), tid, cu(now), cu(nxt))
        torch.cuda.synchronize()
        sn = ostep.shift_sigmas(grid[step], shift)
        sx = ostep.shift_sigmas(grid[step + 1], shift)
        ref = ostep.euler_step(x, v, np.full((1, len(idx)), sn), np.full((1, len(idx)), sx))
        assert np.abs(got.cpu().numpy().astype(np.float64) - ref).max() <= 1e-6 * np.abs(ref).max(), shift


# ---------------------------------------------------------------- a whole denoising step

@pytest.mark.parametrize("mode", ["f32", "bf16", "w8a8"])
def test_denoise_step(mode):
    # input projections -> two blocks -> heads -> Euler update, against the
    # oracle's composition of the same steps (bf16 storage of the packed
    # sequence after the input projections and after the chain, as the
    # library stores them)
    print(f"denoise step {mode}", flush=True)
    from oracle import block as ob
    from oracle import edges as oe
    from oracle import w8a8 as ow
    from oracle import weights_f64
    dtype = "f32" if mode == "f32" else "bf16"
    dims = synth.ModelDims(hidden=512, num_heads=4, head_dim=128, ffn_dim=768, num_tvals=16, dtype=dtype)
    segs = [("text", 23), ("cond", 12, (1, 3, 4)), ("audio", 17), ("video", 60, (2, 5, 6))]
    wl = synth.make_custom(dims, segs, (2, 5, 6), 5, seed=8, batch=2, num_blocks=2)
    L = wl.layout
    e = synth.make_edges(dims, L, batch=2, seed=9)
    k = 4
    grid = (1.0 - np.arange(k) / k).astype(np.float32)
    now, nxt = grid[np.arange(16) // k], grid[np.arange(16) % k]
    cfg, lay, blocks, _ = dv.upload(wl)
    if mode == "w8a8":
        blocks = [m.DeviceBlockW8A8.from_block(b) for b in blocks]
    video, audio = dv.f32(e.video), dv.f32(e.audio)
    m.denoise_step(cfg, lay, blocks, dv.edges_for(e), dv.f32(now), dv.f32(nxt), video, audio, dv.to_device(e.text),
                   flags=m.VALIDATE)
    torch.cuda.synchronize()

    store = (lambda a: a) if dtype == "f32" else ow.round_bf16
    x = store(oe.embed_inputs(e.video, e.audio, e.text.values(), L, e.w_in, e.b_in, e.w_ain, e.b_ain, dims.hidden))
    ws = [weights_f64(b) for b in wl.blocks]
    for bi in range(2):
        for i, w in enumerate(ws):
            x[bi] = ow.block_forward_w8a8(x[bi], L, w, dims) if mode == "w8a8" else ob.block_forward(x[bi], L, w, dims)
    x = store(x)
    v, a = oe.output_heads(x, L, e.gamma, e.beta, e.final_norm_eps, e.w_out, e.b_out, e.w_aout, e.b_aout)
    tv, ta = L.timestep_indices[L.video_indices], L.timestep_indices[L.audio_indices]
    ref_v = ostep.euler_step(e.video, v, np.broadcast_to(now[tv], (2, len(tv))), np.broadcast_to(nxt[tv], (2, len(tv))))
    ref_a = ostep.euler_step(e.audio, a, np.broadcast_to(now[ta], (2, len(ta))), np.broadcast_to(nxt[ta], (2, len(ta))))
    # compare the updates (x' - x): they carry all of the step's arithmetic
    for got, ref, x0, name in ((video, ref_v, e.video, "video"), (audio, ref_a, e.audio, "audio")):
        d_got = to_np64(got) - x0.astype(np.float64)
        d_ref = ref - x0.astype(np.float64)
        if mode == "f32":
            assert rel_l2(d_got, d_ref) <= REL_L2_F32, name
        else:
            assert_close(d_got, d_ref, f"step update {name}", mabs=0.1 if mode == "w8a8" else 5e-2)
    # rows whose timestep value has r = t (the grid's diagonal) stay put
    keep = now[tv] == nxt[tv]
    assert keep.any() and np.array_equal(video.cpu().numpy()[:, keep], e.video[:, keep])
