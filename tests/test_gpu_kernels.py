"""Per-kernel parity of the HIP path against the fp64 oracle (GPU).

Each kernel is called through the C ABI (ctypes binding) on seeded inputs
that span several tiles with a ragged tail, and compared element by element
with the oracle at the bar stated in tests/helpers.py; at the largest sizes
(a projection operand at its 4 GiB limit, a 131k-row attention) on sampled
rows.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

from helpers import REL_L2_F32, assert_close, gpu_available, rel_l2, to_np64
from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth
from oracle import block as ob

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return dv.to_device(synth.Tensor(synth.round_to_bf16_bits(a.astype(np.float32)), "bf16"))


def bf16_vals(a: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(synth.round_to_bf16_bits(a.astype(np.float32))).astype(np.float64)


# ---------------------------------------------------------------- GEMM

# K steps of 64: one, two, three (the pipeline's prologue and clamped tail loads), and longer
@pytest.mark.parametrize("M,N,K", [(300, 512, 384), (1, 256, 64), (260, 256, 128), (257, 512, 192), (513, 768, 640),
                                   (2048, 1024, 512)])
def test_linear_bf16(M, N, K):
    print(f"linear bf16 M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    out = m.linear(bf16_dev(a), bf16_dev(w))
    torch.cuda.synchronize()
    ref = bf16_vals(a) @ bf16_vals(w).T
    got = to_np64(out)
    assert_close(got, ref, "linear")
    # element-level: bf16 rounding of an fp32-accumulated value
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-3)


def test_linear_bf16_operand_at_its_4gib_limit():
    # the A operand one row short of 4 GiB, the largest bf16 projection
    # operand the library takes (its DMA offsets are 32-bit); one row more is
    # refused on the host before any GPU work
    M, N, K = (1 << 18) - 1, 256, 8192
    print(f"linear bf16 at the operand limit M={M} K={K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, 1 << 15):  # drawn in slices: no 8 GiB fp32 temporary
        r1 = min(M, r0 + (1 << 15))
        a[r0:r1] = torch.randn(r1 - r0, K, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    assert M * K * 2 < (1 << 32) <= (M + 1) * K * 2
    out = m.linear(a, w)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 255, 256, 131071, 261887, 261888, M - 1])
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ref = f64(a[sel]) @ f64(w).T
    got = f64(out[sel])
    assert_close(got, ref, "linear at the operand limit")
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-3)
    p = ctypes.c_void_p(a.data_ptr())
    assert m.lib().minih3_linear(0, p, p, p, M + 1, N, K, None) == m.E_UNSUPPORTED


@pytest.mark.parametrize("M,N,K", [(70, 128, 48), (5, 64, 16)])
def test_linear_f32(M, N, K):
    rng = np.random.default_rng(1)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    out = m.linear(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    assert rel_l2(to_np64(out), ref) <= REL_L2_F32


# ---------------------------------------------------------------- AdaLN

def small_bf16_dims(**kw):
    d = dict(hidden=512, num_heads=4, head_dim=128, ffn_dim=768, num_tvals=8, dtype="bf16")
    d.update(kw)
    return synth.ModelDims(**d)


def small_workload(dims, pads=13, seed=0, batch=1, segs=None, grid=(3, 5, 7)):
    segs = segs or [("text", 37), ("cond", 20, (1, 4, 5)), ("audio", 29), ("video", 105, grid)]
    return synth.make_custom(dims, segs, grid, pads, seed=seed, batch=batch)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("which", [0, 1])
def test_adaln_modulate(dtype, which):
    dims = small_bf16_dims(dtype=dtype, hidden=5376 if dtype == "bf16" else 512)
    # which=1: 2 x 205 rows, so the last workgroup of four rows is partly empty
    wl = small_workload(dims, batch=2, pads=13 + which)
    cfg, lay, blocks, x = dv.upload(wl)
    y = m.adaln_modulate(cfg, lay, x, blocks[0].adaln_table, which)
    torch.cuda.synchronize()
    L = wl.layout
    tab = wl.blocks[0].adaln_table.astype(np.float64)
    for b in range(2):
        ref = ob.adaln(wl.x.values()[b], tab, L.token_tags, L.timestep_indices, which, dims.norm_eps)
        got = to_np64(y[b])
        if dtype == "bf16":
            assert_close(got, ref, "adaln")
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)
        else:
            assert rel_l2(got, ref) <= REL_L2_F32


# ---------------------------------------------------------------- RMSNorm + RoPE

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("heads", [4, 3])  # two heads per workgroup, and one (odd head count)
def test_qk_norm_rope(dtype, heads):
    dims = small_bf16_dims(dtype=dtype, num_heads=heads)
    wl = small_workload(dims, batch=2)
    cfg, lay, blocks, _ = dv.upload(wl)
    B, S, H, hd = 2, wl.layout.seq_len, dims.num_heads, dims.head_dim
    W = H * hd
    rng = np.random.default_rng(3)
    qkv = (rng.standard_normal((B, S, 3 * W)) * 1.7).astype(np.float32)
    if dtype == "bf16":
        qkv_dev, qkv64 = bf16_dev(qkv), bf16_vals(qkv)
    else:
        qkv_dev, qkv64 = torch.from_numpy(qkv).cuda(), qkv.astype(np.float64)
    q, k, vt = m.qk_norm_rope(cfg, lay, qkv_dev, blocks[0].q_norm, blocks[0].k_norm)
    torch.cuda.synchronize()
    st = lay.seq_stride
    pos = wl.layout.position_ids
    gq = wl.blocks[0].q_norm.astype(np.float64)
    gk = wl.blocks[0].k_norm.astype(np.float64)
    for b in range(B):
        qr = ob.rope_3d(ob.rms_norm_heads(qkv64[b, :, :W].reshape(S, H, hd), gq, 1e-5), pos, 16, 1e4)
        kr = ob.rope_3d(ob.rms_norm_heads(qkv64[b, :, W:2 * W].reshape(S, H, hd), gk, 1e-5), pos, 16, 1e4)
        v = qkv64[b, :, 2 * W:].reshape(S, H, hd)
        got_q = to_np64(q[b]).transpose(1, 0, 2)  # [stride, H, hd]
        got_k = to_np64(k[b]).transpose(1, 0, 2)
        got_v = to_np64(vt[b]).transpose(2, 0, 1)  # [stride, H, hd]
        if dtype == "bf16":
            assert_close(got_q[:S], qr, "q_rot")
            assert_close(got_k[:S], kr, "k_rot")
            assert np.array_equal(got_v[:S], v)          # a pure transpose: exact
        else:
            assert rel_l2(got_q[:S], qr) <= REL_L2_F32 and rel_l2(got_k[:S], kr) <= REL_L2_F32
            assert np.array_equal(got_v[:S], v)
        assert np.all(got_q[S:] == 0) and np.all(got_k[S:] == 0) and np.all(got_v[S:] == 0)


# ---------------------------------------------------------------- attention

def attention_case(S, H, pad_rows, seed, B=1, dtype="bf16", sharp=1.0):
    rng = np.random.default_rng(seed)
    hd = 128
    st = (S + 63) // 64 * 64
    tags = np.ones(S, np.int32)
    tags[list(pad_rows)] = -1
    q = rng.standard_normal((B, H, st, hd)) * sharp
    k = rng.standard_normal((B, H, st, hd))
    v = rng.standard_normal((B, H, st, hd))
    if dtype == "bf16":
        qd, kd = bf16_dev(q), bf16_dev(k)
        vtd = bf16_dev(np.ascontiguousarray(v.transpose(0, 1, 3, 2)))
        q, k, v = bf16_vals(q), bf16_vals(k), bf16_vals(v)
    else:
        qd, kd = torch.from_numpy(q.astype(np.float32)).cuda(), torch.from_numpy(k.astype(np.float32)).cuda()
        vtd = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 1, 3, 2)).astype(np.float32)).cuda()
        q, k, v = (a.astype(np.float32).astype(np.float64) for a in (q, k, v))
    dims = synth.ModelDims(hidden=256, num_heads=H, head_dim=hd, ffn_dim=256, dtype=dtype)
    cfg = dv.config_for(dims)
    z = np.zeros(S, np.int32)
    lay = m.DeviceLayout(B, tags, z, np.zeros((S, 3), np.int32), z[:0], z[:0], z[:0])
    return cfg, lay, (qd, kd, vtd), (q, k, v), tags


@pytest.mark.parametrize("S,pads", [(64, []), (200, [3, 77, 150, 151, 199]), (517, list(range(480, 517))),
                                    (700, [0] + list(range(256, 320))), (1000, list(range(100, 900)))])
def test_attention_doc_mask(S, pads):
    print(f"attention S={S} pads={len(pads)}", flush=True)
    H = 3
    cfg, lay, (qd, kd, vtd), (q, k, v), tags = attention_case(S, H, pads, seed=S, B=2, sharp=1.0)
    out = m.attention_headmajor(cfg, lay, qd, kd, vtd)
    torch.cuda.synchronize()
    doc = ob.doc_ids(tags)
    for b in range(2):
        ref = ob.attention_doc_masked(q[b, :, :S].transpose(1, 0, 2), k[b, :, :S].transpose(1, 0, 2),
                                      v[b, :, :S].transpose(1, 0, 2), doc, 1 / math.sqrt(128))
        got = to_np64(out[b]).reshape(S, H, 128)
        assert_close(got, ref, f"attention b={b}")


@pytest.mark.parametrize("S,pads", [(300, [5, 6, 299]), (129, [])])
def test_attention_sharp(S, pads):
    # peaked softmax: a wrong mask, key order or rotation would show
    H = 2
    cfg, lay, (qd, kd, vtd), (q, k, v), tags = attention_case(S, H, pads, seed=7, sharp=4.0)
    out = m.attention_headmajor(cfg, lay, qd, kd, vtd)
    torch.cuda.synchronize()
    ref = ob.attention_doc_masked(q[0, :, :S].transpose(1, 0, 2), k[0, :, :S].transpose(1, 0, 2),
                                  v[0, :, :S].transpose(1, 0, 2), ob.doc_ids(tags), 1 / math.sqrt(128))
    assert_close(to_np64(out[0]).reshape(S, H, 128), ref, "sharp attention")


def test_attention_long_sequence_sampled_queries():
    # four times the clip-scale sequence, a ragged end, padding rows at the
    # end and two inside; queries sampled at tile edges, in both documents
    S, H = 131072 + 37, 2
    print(f"attention long sequence S={S}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(6)
    q, k, v = (torch.randn(1, S, H, 128, device="cuda", generator=g).mul(s).to(torch.bfloat16)
               for s in (2.0, 1.0, 1.0))
    tags = np.zeros(S, np.int32)
    tags[-1000:] = -1
    tags[[5, 70000]] = -1
    cfg = dv.config_for(synth.ModelDims(hidden=256, num_heads=H, head_dim=128, ffn_dim=256, dtype="bf16"))
    z = np.zeros(S, np.int32)
    lay = m.DeviceLayout(1, tags, z, np.zeros((S, 3), np.int32), z[:0], z[:0], z[:0])
    out = m.attention_packed(cfg, lay, q, k, v)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 5, 63, 64, 4095, 70000, 131071, 131072, S - 1001, S - 1000, S - 1],
                                     rng.integers(0, S, 21)]))
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ref = ob.attention_doc_masked(f64(q[0]), f64(k[0]), f64(v[0]), ob.doc_ids(tags), 1 / math.sqrt(128), rows=rows)
    got = f64(out[0, rows]).reshape(len(rows), H, 128)
    assert_close(got, ref, "attention, long sequence")


def test_attention_f32():
    S, H = 150, 2
    cfg, lay, (qd, kd, vtd), (q, k, v), tags = attention_case(S, H, [10, 149], seed=2, dtype="f32")
    out = m.attention_headmajor(cfg, lay, qd, kd, vtd)
    torch.cuda.synchronize()
    ref = ob.attention_doc_masked(q[0, :, :S].transpose(1, 0, 2), k[0, :, :S].transpose(1, 0, 2),
                                  v[0, :, :S].transpose(1, 0, 2), ob.doc_ids(tags), 1 / math.sqrt(128))
    assert rel_l2(to_np64(out[0]).reshape(S, H, 128), ref) <= REL_L2_F32


def packed_inputs(q, k, v, S, dtype):
    """[B, H, stride, hd] values -> device q, k, v [B, S, H, hd] (exact)."""
    outs = []
    for a in (q, k, v):
        p = np.ascontiguousarray(a[:, :, :S].transpose(0, 2, 1, 3))
        outs.append(bf16_dev(p) if dtype == "bf16" else torch.from_numpy(p.astype(np.float32)).cuda())
    return outs


@pytest.mark.parametrize("S,pads,B,dtype,sharp", [(200, [3, 77, 150, 151, 199], 2, "bf16", 1.0),
                                                  (517, list(range(480, 517)), 1, "bf16", 1.0),
                                                  (700, [0] + list(range(256, 320)), 1, "bf16", 4.0),
                                                  (1, [], 1, "bf16", 1.0), (65, [64], 1, "bf16", 1.0),
                                                  (150, [10, 149], 1, "f32", 1.0)])
def test_attention_packed_entry(S, pads, B, dtype, sharp):
    # the boundary entry point: packed [B, S, H, hd] q / k / v after norm and
    # rotary, staged by the library into the kernels' layouts
    print(f"attention packed entry S={S} pads={len(pads)} B={B} {dtype}", flush=True)
    H = 3
    cfg, lay, (qd, kd, vtd), (q, k, v), tags = attention_case(S, H, pads, seed=S + 11, B=B, dtype=dtype,
                                                              sharp=sharp)
    qp, kp, vp = packed_inputs(q, k, v, S, dtype)
    out = m.attention_packed(cfg, lay, qp, kp, vp)
    ref_hm = m.attention_headmajor(cfg, lay, qd, kd, vtd)
    torch.cuda.synchronize()
    # the staging is a copy: the two entries give the same bits
    assert torch.equal(out, ref_hm)
    doc = ob.doc_ids(tags)
    for b in range(B):
        ref = ob.attention_doc_masked(q[b, :, :S].transpose(1, 0, 2), k[b, :, :S].transpose(1, 0, 2),
                                      v[b, :, :S].transpose(1, 0, 2), doc, 1 / math.sqrt(128))
        got = to_np64(out[b]).reshape(S, H, 128)
        if dtype == "bf16":
            assert_close(got, ref, f"attention packed b={b}")
        else:
            assert rel_l2(got, ref) <= REL_L2_F32


def test_attention_packed_entry_errors():
    S, H = 100, 2
    cfg, lay, _, (q, k, v), _ = attention_case(S, H, [5], seed=3)
    qp, kp, vp = packed_inputs(q, k, v, S, "bf16")
    with pytest.raises(m.Minih3Error) as e:
        m.attention_packed(cfg, lay, qp, kp, vp, flags=m.ASSUME_PADLESS | m.VALIDATE)
    assert e.value.status == m.E_NEEDS_MASK
    ws = m.alloc_workspace(m.attention_workspace_bytes(cfg, 1, S) - 1)
    with pytest.raises(m.Minih3Error) as e:
        m.attention_packed(cfg, lay, qp, kp, vp, workspace=ws)
    assert e.value.status == m.E_WORKSPACE
    with pytest.raises(m.Minih3Error) as e:
        m.attention_packed(cfg, lay, qp, kp, vp, out=qp.view(1, S, H * 128))
    assert e.value.status == m.E_ARG


def test_attention_padless_flag_matches_masked_path_bit_exact():
    S, H = 333, 2
    cfg, lay, (qd, kd, vtd), _, _ = attention_case(S, H, [], seed=4)
    a = m.attention_headmajor(cfg, lay, qd, kd, vtd)
    b = m.attention_headmajor(cfg, lay, qd, kd, vtd, flags=m.ASSUME_PADLESS | m.VALIDATE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    cfg, lay, (qd, kd, vtd), _, _ = attention_case(S, H, [7], seed=4)
    with pytest.raises(m.Minih3Error) as e:
        m.attention_headmajor(cfg, lay, qd, kd, vtd, flags=m.ASSUME_PADLESS | m.VALIDATE)
    assert e.value.status == m.E_NEEDS_MASK
