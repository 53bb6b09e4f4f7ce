"""Parity of the rotated W8A8 INT8 path against the oracle (GPU).

The int8 codes and their scales are integers / float32 values decided by
float32 arithmetic in a fixed order, so they are compared bit-exactly; the
product accumulates exactly in int32, so the bf16 output is checked element
by element against the exact dequantized value (one fp32 dequantization and
one bf16 rounding apart).
"""
import numpy as np
import pytest
import torch

from helpers import gpu_available, rel_l2
from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth
from oracle import w8a8 as ow

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def bf16_pair(a: np.ndarray):
    t = synth.Tensor(synth.round_to_bf16_bits(a.astype(np.float32)), "bf16")
    return dv.to_device(t), synth.bf16_bits_to_f32(t.data)


def rows(M, K, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * scale).astype(np.float32)
    if M > 3:
        x[1] = 0.0                 # all-zero row: codes 0, scale 0
        x[2] = 0.0
        x[2, K // 3] = -7.5        # one large value
    return x


@pytest.mark.parametrize("M,K", [(5, 128), (33, 384), (300, 5376), (17, 7168), (9, 14336)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rotate_quantize_bit_exact(M, K, dtype):
    print(f"rotate_quantize {dtype} M={M} K={K}", flush=True)
    x = rows(M, K, M + K, scale=2.0)
    if dtype == "bf16":
        xd, xv = bf16_pair(x)
    else:
        xd, xv = torch.from_numpy(x).cuda(), x
    q, sc = m.rotate_quantize(xd)
    torch.cuda.synchronize()
    rq, rs = ow.rotate_quantize(xv)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.all(q[1].cpu().numpy() == 0) and sc[1].item() == 0.0


def check_linear(qa, sa, qw, sw, out):
    acc = ow.int_matmul(qa, qw).astype(np.float64)
    ref = acc * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    got = out.float().cpu().numpy().astype(np.float64)
    tol = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (int(bad.sum()), float(np.abs(got - ref).max()))


# K steps of 128: one, two, five, eight; ragged M
@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (300, 512, 256), (513, 768, 640), (2048, 1024, 1024)])
def test_linear_w8a8(M, N, K):
    print(f"linear_w8a8 M={M} N={N} K={K}", flush=True)
    xd, xv = bf16_pair(rows(M, K, 1))
    wd, wv = bf16_pair(rows(N, K, 2, scale=0.02))
    qa, sa = m.rotate_quantize(xd)
    qw, sw = m.rotate_quantize(wd)
    out = m.linear_w8a8(qa, sa, qw, sw)
    torch.cuda.synchronize()
    # the codes are the oracle's (bit-exact above); the product is checked against their exact value
    rqa, rsa = ow.rotate_quantize(xv)
    rqw, rsw = ow.rotate_quantize(wv)
    assert np.array_equal(qa.cpu().numpy(), rqa) and np.array_equal(qw.cpu().numpy(), rqw)
    check_linear(rqa, rsa, rqw, rsw, out)
    # and the W8A8 result tracks the bf16 product within the quantization error
    ref = xv.astype(np.float64) @ wv.astype(np.float64).T
    got = out.float().cpu().numpy()
    assert np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30) < 3e-2


def test_linear_w8a8_full_qkv_shape_sampled_rows():
    # the QKV projection of the clip-scale block: 32768 x 21504 x 5376
    print("linear_w8a8 full QKV shape", flush=True)
    M, N, K = 32768, 21504, 5376
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    qa, sa = m.rotate_quantize(x)
    qw, sw = m.rotate_quantize(w)
    out = m.linear_w8a8(qa, sa, qw, sw)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 255, 256, 4097, 20000, 32766, 32767])
    xs = x[sel].float().cpu().numpy()
    rqa, rsa = ow.rotate_quantize(xs)
    assert np.array_equal(qa[sel].cpu().numpy(), rqa)
    rqw, rsw = ow.rotate_quantize(w.float().cpu().numpy())
    assert np.array_equal(qw.cpu().numpy(), rqw)
    check_linear(rqa, rsa, rqw, rsw, out[sel])


# ---------------------------------------------------------------- the W8A8 block
#
# The block's W8A8 results are compared with the W8A8 oracle at relative L2
# <= 1e-2 (the bf16 bar) and max-abs <= 0.1: the int8 codes of a projection
# are decided by its bf16 input, and where the GPU's and the oracle's bf16
# activations differ by one ulp (different summation orders upstream) a code
# can move by one step, amax / 127 -- about eight times the ulp that caused
# it -- so single output elements may differ by a few bf16 ulps where the
# plain block's differ by one. The integer product itself is checked exactly
# by the tests above.
W8A8_BLOCK_MAX_ABS = 0.1

def w8a8_block_case(dims, segs, grid, pads, seed, batch):
    wl = synth.make_custom(dims, segs, grid, pads, seed=seed, batch=batch)
    cfg, lay, blocks, x = dv.upload(wl)
    qb = [m.DeviceBlockW8A8.from_block(b) for b in blocks]
    out = m.block_forward_w8a8(cfg, lay, qb, x, flags=m.VALIDATE)
    torch.cuda.synchronize()
    return wl, x, out


@pytest.mark.parametrize("pads", [0, 13])
def test_block_w8a8_small(pads):
    print(f"block w8a8 small pads={pads}", flush=True)
    from oracle import weights_f64
    from helpers import assert_close, to_np64
    dims = synth.ModelDims(hidden=512, num_heads=4, head_dim=128, ffn_dim=768, num_tvals=8, dtype="bf16")
    segs = [("text", 37), ("cond", 20, (1, 4, 5)), ("audio", 29), ("video", 105, (3, 5, 7))]
    wl, x, out = w8a8_block_case(dims, segs, (3, 5, 7), pads, seed=pads, batch=2)
    w = weights_f64(wl.blocks[0])
    got = to_np64(out)
    for b in range(2):
        ref = ow.block_forward_w8a8(wl.x.values()[b], wl.layout, w, dims)
        assert_close(got[b], ref, f"w8a8 block, item {b}", mabs=W8A8_BLOCK_MAX_ABS)
    # padding rows leave the block bit for bit
    pad = wl.layout.token_tags == -1
    assert np.array_equal(got[:, pad], wl.x.values()[:, pad])


@pytest.mark.parametrize("hidden,heads,ffn", [(512, 4, 768), (5376, 56, 14336)])
def test_block_w8a8_adaln_writes_the_same_codes(hidden, heads, ffn):
    # In the W8A8 block the AdaLN kernels write the rotated int8 rows of the
    # next projection themselves; asking for the bf16 AdaLN rows as taps
    # takes the separate AdaLN -> rotate/quantize route instead. Both must give
    # the same block output bit for bit (the same bf16 values, the same
    # rotation and quantization arithmetic).
    print(f"w8a8 fused AdaLN quantization hidden={hidden}", flush=True)
    dims = synth.ModelDims(hidden=hidden, num_heads=heads, head_dim=128, ffn_dim=ffn, num_tvals=8, dtype="bf16")
    segs = [("text", 21), ("audio", 30), ("video", 90, (2, 5, 9))]
    wl = synth.make_custom(dims, segs, (2, 5, 9), 7, seed=4, batch=2)
    cfg, lay, blocks, x = dv.upload(wl)
    qb = [m.DeviceBlockW8A8.from_block(b) for b in blocks]
    fused = m.block_forward_w8a8(cfg, lay, qb, x)
    B, S = lay.batch, lay.seq_len
    taps = dict(adaln1=torch.empty(B, S, hidden, dtype=torch.bfloat16, device="cuda"),
                adaln2=torch.empty(B, S, hidden, dtype=torch.bfloat16, device="cuda"))
    separate = m.block_forward_w8a8(cfg, lay, qb, x, taps=taps)
    torch.cuda.synchronize()
    assert torch.equal(fused, separate)


def test_block_w8a8_gate_zero_is_identity():
    dims = synth.ModelDims(hidden=512, num_heads=4, head_dim=128, ffn_dim=768, num_tvals=8, dtype="bf16")
    wl = synth.make_custom(dims, [("text", 40), ("video", 90, (2, 5, 9))], (2, 5, 9), 6, seed=3)
    wl.blocks[0].adaln_table[:, :, 2] = 0.0
    wl.blocks[0].adaln_table[:, :, 5] = 0.0
    cfg, lay, blocks, x = dv.upload(wl)
    qb = [m.DeviceBlockW8A8.from_block(b) for b in blocks]
    out = m.block_forward_w8a8(cfg, lay, qb, x)
    torch.cuda.synchronize()
    assert torch.equal(out, x)


def code_flips(x_gpu: np.ndarray, x_ref: np.ndarray):
    """How the GPU's bf16 projection inputs and the oracle's differ, and what
    that does to the int8 codes: (fraction of differing bf16 elements,
    fraction of rows whose scale differs, fraction of differing codes,
    largest code change)."""
    qg, sg = ow.rotate_quantize(x_gpu)
    qr, sr = ow.rotate_quantize(x_ref)
    dq = np.abs(qg.astype(np.int32) - qr.astype(np.int32))
    return (float(np.mean(x_gpu != x_ref)), float(np.mean(sg != sr)), float(np.mean(dq > 0)), int(dq.max()))


def test_block_w8a8_full_width():
    # the clip-scale block's widths (hidden 5376, 56 x 128 heads, FFN 14336) on 300 rows
    print("block w8a8 full width", flush=True)
    from oracle import block as ob
    from oracle import weights_f64
    from helpers import assert_close, assert_close_bf16_storage, to_np64
    dims = synth.ModelDims(num_tvals=8)
    segs = [("text", 40), ("audio", 36), ("video", 216, (2, 9, 12))]
    wl = synth.make_custom(dims, segs, (2, 9, 12), 8, seed=5, batch=1)
    cfg, lay, blocks, x = dv.upload(wl)
    qb = [m.DeviceBlockW8A8.from_block(b) for b in blocks]
    B, S, D = 1, lay.seq_len, dims.hidden
    W, F = dims.num_heads * dims.head_dim, dims.ffn_dim
    bf = lambda *sh: torch.empty(*sh, dtype=torch.bfloat16, device="cuda")
    taps = dict(adaln1=bf(B, S, D), attn_o=bf(B, S, W), attn_proj=bf(B, S, D), adaln2=bf(B, S, D),
                ffn_h=bf(B, S, F), ffn_out=bf(B, S, D))
    out = m.block_forward_w8a8(cfg, lay, qb, x, flags=m.VALIDATE, taps=taps)
    # the library's codes of each projection input
    gq = {k: m.rotate_quantize(taps[k][0]) for k in ("adaln1", "attn_o", "adaln2", "ffn_h")}
    torch.cuda.synchronize()
    w = weights_f64(wl.blocks[0])
    t = {k: to_np64(v[0]) for k, v in taps.items()}

    # 1. Each projection on the kernel's own bf16 inputs: the library's codes
    # equal the oracle's bit for bit, and the product (and the epilogue that
    # consumes it) equals the oracle's exact integer product dequantized
    for k in gq:
        rq, rs = ow.rotate_quantize(t[k])
        assert np.array_equal(gq[k][0].cpu().numpy(), rq), k
        assert np.array_equal(gq[k][1].cpu().numpy().view(np.uint32), rs.view(np.uint32)), k
    check_own = {"attn_proj": ow.linear_w8a8(t["attn_o"], w["w_out"]),
                 "ffn_out": ow.linear_w8a8(t["ffn_h"], w["w_down"])}
    gu = ow.linear_w8a8(t["adaln2"], w["w_gate_up"])
    check_own["ffn_h"] = ob.silu(gu[:, :F]) * gu[:, F:]
    for k, want in check_own.items():
        r = assert_close_bf16_storage(t[k], want, f"w8a8 {k} on its own inputs")
        print(f"w8a8 {k} on the kernel's own inputs: rel_l2={r[0]:.3e} max_abs={r[1]:.3e}", flush=True)

    # 2. End to end against the W8A8 oracle, whose projection inputs are its
    # own fp64 activations rounded to bf16. Where the two bf16 activations
    # differ (summation order upstream), codes change: when a row's largest
    # element moves by one bf16 ulp its scale moves by up to 2^-8 and every
    # code of the row whose scaled value sits within that much of a rounding
    # boundary changes by one step.
    ref, rt = ow.block_forward_w8a8(wl.x.values()[0], wl.layout, w, dims, taps=True)
    for k in ("adaln1", "attn_o", "adaln2", "ffn_h"):
        f_el, f_row, f_code, dmax = code_flips(t[k], rt[k])
        print(f"w8a8 flips {k}: bf16 elements differing {f_el:.4f}, row scales differing {f_row:.4f}, "
              f"codes differing {f_code:.5f}, largest code change {dmax}", flush=True)
    # A product whose input codes flipped differs from the oracle's by about
    # its quantization error: bound it by the bf16 bar plus twice the
    # oracle's own quantization error of that product (W8A8 against the
    # exact product of the same bf16 input)
    exact = {"attn_proj": rt["attn_o"] @ w["w_out"].T, "ffn_out": rt["ffn_h"] @ w["w_down"].T}
    for k in ("attn_proj", "ffn_out"):
        r = rel_l2(t[k], rt[k])
        q_err = rel_l2(rt[k], exact[k])
        print(f"w8a8 {k} end to end: rel_l2={r:.3e} max_abs={np.abs(t[k] - rt[k]).max():.3e}; the oracle's own "
              f"quantization error {q_err:.3e}", flush=True)
        assert r <= 1e-2 + 2 * q_err, (k, r, q_err)
    r, mx = assert_close(to_np64(out)[0], ref, "w8a8 block, full width", mabs=W8A8_BLOCK_MAX_ABS)
    print(f"w8a8 block full width: rel_l2={r:.3e} max_abs={mx:.3e} (plain fp64 block: rel_l2 "
          f"{rel_l2(to_np64(out)[0], ob.block_forward(wl.x.values()[0], wl.layout, w, dims)):.3e})", flush=True)
