"""Pins of the rotated W8A8 oracle against the Hadamard matrix of a library,
orthogonality, exact integer arithmetic, the quantization error bound and
hand-worked values (CPU only).

A wrong butterfly, a missing normalisation, a rotation applied to one
operand only, a wrong rounding or clamp, or a scale from the wrong axis each
fail at least one of these.
"""
import itertools

import numpy as np
from scipy.linalg import hadamard

from oracle import w8a8 as ow


def test_fwht_equals_scipy_hadamard_blockwise():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 384)).astype(np.float32)
    H = hadamard(128).astype(np.float64) / np.sqrt(128.0)
    ref = np.concatenate([x[:, 128 * b:128 * (b + 1)].astype(np.float64) @ H for b in range(3)], axis=1)
    got = ow.fwht_blocks_f32(x).astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()


def test_fwht_of_unit_vectors_is_a_signed_column_exactly():
    # e_k maps to column k of H / sqrt(128): every entry is +-1/sqrt(128) in float32
    for k in (0, 1, 77, 127):
        e = np.zeros((1, 128), np.float32)
        e[0, k] = 1.0
        got = ow.fwht_blocks_f32(e)[0]
        col = hadamard(128)[:, k].astype(np.float32) * ow.INV_SQRT_BLOCK
        assert np.array_equal(got, col)


def test_fwht_is_orthogonal_and_an_involution():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 256)).astype(np.float32)
    y = ow.fwht_blocks_f32(x)
    # Parseval per 128-block, and H H = I
    for b in range(2):
        sl = slice(128 * b, 128 * (b + 1))
        assert np.allclose((y[:, sl].astype(np.float64) ** 2).sum(1), (x[:, sl].astype(np.float64) ** 2).sum(1),
                           rtol=1e-5)
    assert np.abs(ow.fwht_blocks_f32(y) - x).max() <= 1e-5


def test_rotation_preserves_products():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 384))
    w = rng.standard_normal((6, 384))
    lhs = ow.fwht_blocks_f32(x).astype(np.float64) @ ow.fwht_blocks_f32(w).astype(np.float64).T
    assert np.abs(lhs - x @ w.T).max() <= 1e-4 * np.abs(x @ w.T).max()


def test_quantize_hand_worked_and_bounds():
    # amax = 2.54 (float32): 127 / 2.54 rounds to exactly 50 in float32; then 1.0 -> 50, -2.54 -> -127,
    # 0.01 * 50 rounds to 0.5 -> 0 (ties to even), 0.03 * 50 rounds to 1.5 -> 2 (ties to even)
    v = np.array([[1.0, -2.54, 0.01, 0.03]], np.float32)
    q, s = ow.quantize_rows_f32(v)
    assert np.float32(127.0) / np.float32(2.54) == np.float32(50.0)
    assert q[0].tolist() == [50, -127, 0, 2]
    assert s[0] == np.float32(2.54) / np.float32(127.0)
    # the round-trip error is at most half a step, and zero rows stay zero
    rng = np.random.default_rng(3)
    r = rng.standard_normal((20, 128)).astype(np.float32) * 3
    q, s = ow.quantize_rows_f32(r)
    assert np.all(np.abs(q.astype(np.float64) * s[:, None] - r) <= 0.5 * s[:, None] * (1 + 1e-5) + 1e-7)
    assert np.all(np.abs(q).max(axis=1) == 127)
    qz, sz = ow.quantize_rows_f32(np.zeros((2, 128), np.float32))
    assert np.all(qz == 0) and np.all(sz == 0)


def test_int_matmul_brute_force():
    rng = np.random.default_rng(4)
    a = rng.integers(-127, 128, (3, 5)).astype(np.int8)
    b = rng.integers(-127, 128, (4, 5)).astype(np.int8)
    got = ow.int_matmul(a, b)
    for i, j in itertools.product(range(3), range(4)):
        assert got[i, j] == sum(int(a[i, k]) * int(b[j, k]) for k in range(5))
    # the worst case of a 14336-deep product stays inside int32
    assert 14336 * 127 * 127 < 2 ** 31


def test_linear_w8a8_within_the_quantization_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 512))
    w = rng.standard_normal((16, 512)) * 0.02
    y = ow.linear_w8a8(x, w)
    ref = x @ w.T
    xr, wr = ow.fwht_blocks_f32(x).astype(np.float64), ow.fwht_blocks_f32(w).astype(np.float64)
    _, sx = ow.rotate_quantize(x)
    _, sw = ow.rotate_quantize(w)
    ex, ew = 0.5 * sx.astype(np.float64), 0.5 * sw.astype(np.float64)
    bound = (np.abs(xr).sum(1)[:, None] * ew[None, :] + ex[:, None] * np.abs(wr).sum(1)[None, :]
             + 512 * ex[:, None] * ew[None, :]) * (1 + 1e-3) + 1e-6
    assert np.all(np.abs(y - ref) <= bound)
    # and the error is small in the usual sense
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 2e-2


def test_round_bf16_values():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1;
    # 1 + 3 * 2^-8 ties up to 1 + 2^-6 (even mantissa); 3.0 is exact
    got = ow.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.0, -1.5]))
    assert got.tolist() == [1.0, 1 + 2.0 ** -6, 3.0, -1.5]


def test_w8a8_block_tracks_the_plain_block():
    # the W8A8 block differs from the plain block only by the quantization of
    # the four projections: with gate 0 both are the identity, and otherwise
    # they agree to the quantization error
    from oracle import block as ob
    from oracle import weights_f64
    from joint_video_audio_amd import synth
    dims = synth.ModelDims(hidden=256, num_heads=2, head_dim=128, ffn_dim=384, num_tvals=4, dtype="bf16")
    segs = [("text", 7), ("audio", 5), ("video", 24, (2, 3, 4))]
    wl = synth.make_custom(dims, segs, (2, 3, 4), 3, seed=0)
    w = weights_f64(wl.blocks[0])
    x = wl.x.values()[0]
    y8 = ow.block_forward_w8a8(x, wl.layout, w, dims)
    y = ob.block_forward(x, wl.layout, w, dims)
    rel = np.linalg.norm(y8 - y) / np.linalg.norm(y - x)
    assert rel < 5e-2, rel  # relative to the block's own change of x
    w0 = dict(w)
    w0["adaln_table"] = w["adaln_table"].copy()
    w0["adaln_table"][:, :, 2] = 0.0
    w0["adaln_table"][:, :, 5] = 0.0
    assert np.array_equal(ow.block_forward_w8a8(x, wl.layout, w0, dims), x)


def test_codes_equal_an_fp64_hadamard_away_from_rounding_boundaries():
    # The oracle fixes a float32 butterfly order; the codes it decides must be
    # those of the exact rotation (scipy's Hadamard matrix in float64, exact
    # division and rounding) wherever the exact scaled value v * 127 / amax
    # lies farther from a rounding boundary (x.5) than float32 arithmetic can
    # move it: 7 butterfly stages, the normalisation, the division and the
    # product each err by at most 2^-24 relative, so |t| <= 127 moves by less
    # than 127 * 12 * 2^-24 < 1e-4.
    H = hadamard(128).astype(np.float64) / np.sqrt(128.0)
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((256, 5376)) * rng.uniform(0.1, 10.0, (256, 1))).astype(np.float32)
    x[3, 100] = 40.0  # a row with one dominant value
    q, s = ow.rotate_quantize(x)
    xr = np.concatenate([x[:, 128 * b:128 * (b + 1)].astype(np.float64) @ H for b in range(5376 // 128)], axis=1)
    amax = np.abs(xr).max(axis=1, keepdims=True)
    t = xr * (127.0 / amax)
    q64 = np.clip(np.rint(t), -127, 127)
    near = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
    differ = q.astype(np.float64) != q64
    assert not np.any(differ & ~near), int((differ & ~near).sum())
    assert differ.sum() <= near.sum()
    # the scales are amax / 127 of the exact rotation to float32 accuracy
    assert np.all(np.abs(s.astype(np.float64) - amax[:, 0] / 127.0) <= 1e-6 * amax[:, 0] / 127.0)
