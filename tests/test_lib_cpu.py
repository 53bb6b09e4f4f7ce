"""The C-ABI library loads and exports every symbol include/minih3.h declares
(CPU only: host-side entry points that enqueue no GPU work)."""
import ctypes
import os
import re

import pytest

from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "minih3.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(minih3_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libminih3.so not built")
    # RTLD_NOW: every symbol the library references must resolve (a kernel
    # whose host launch stub was not emitted shows up here)
    lib = ctypes.CDLL(m.LIB_PATH, mode=os.RTLD_NOW)
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m.EXPORTED)


def test_host_side_queries_and_argument_errors():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libminih3.so not built")
    assert m.status_string(m.E_NEEDS_MASK).startswith("layout")
    cfg = dv.config_for(synth.workload_dims("clip32k"))
    nbytes = m.workspace_bytes(cfg, 1, 32768)
    # the workspace holds at least the qkv, q/k/v^T and attention buffers in bf16
    assert nbytes > 32768 * (3 * 7168 + 3 * 7168 + 7168) * 2
    assert m.attention_workspace_bytes(cfg, 1, 100) >= 16 * 2
    lib = m.lib()
    bad = m.Config(**{f: getattr(cfg, f) for f, _ in m.Config._fields_})
    bad.head_dim = 64
    n = ctypes.c_size_t(0)
    assert lib.minih3_workspace_bytes(ctypes.byref(bad), 1, 10, ctypes.byref(n)) == m.E_UNSUPPORTED
    assert lib.minih3_block_forward(None, None, None, 1, None, None, None, 0, 0, None, None) == m.E_ARG
    # a valid call shape with a too-small workspace is refused before any GPU work
    L = m._Layout(1, 8, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), None, 0, None, 0, None, 0)
    bw = (m._BlockWeights * 1)(m._BlockWeights(*[ctypes.c_void_p(16)] * 7))
    s = lib.minih3_block_forward(ctypes.byref(cfg), ctypes.byref(L), bw, 1, ctypes.c_void_p(16),
                                 ctypes.c_void_p(32), ctypes.c_void_p(64), 10, 0, None, None)
    assert s == m.E_WORKSPACE
    assert lib.minih3_linear(0, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 4, 100, 64,
                             None) == m.E_UNSUPPORTED
    # bf16 projection operands above 4 GiB are refused before any GPU work
    assert lib.minih3_linear(0, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 300000, 256, 7168,
                             None) == m.E_UNSUPPORTED
    L_big = m._Layout(1, 160000, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), None, 0, None, 0,
                      None, 0)
    s = lib.minih3_block_forward(ctypes.byref(cfg), ctypes.byref(L_big), bw, 1, ctypes.c_void_p(16),
                                 ctypes.c_void_p(32), ctypes.c_void_p(64), 10, 0, None, None)
    assert s == m.E_UNSUPPORTED


def test_conditioning_host_side_checks():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libminih3.so not built")
    lib = m.lib()
    tc = m.TimeConfig(256, 5376, 2688, 1.0e4)
    n = ctypes.c_size_t(0)
    assert lib.minih3_time_embed_workspace_bytes(ctypes.byref(tc), 64, ctypes.byref(n)) == m.OK
    # the hidden activations and eight split-K partial sums, fp32
    assert n.value >= 64 * 5376 * 4 + 8 * 64 * 2688 * 4
    bad = m.TimeConfig(200, 5376, 2688, 1.0e4)
    assert lib.minih3_time_embed_workspace_bytes(ctypes.byref(bad), 64, ctypes.byref(n)) == m.E_UNSUPPORTED
    mlp = m._TimeMLP(ctypes.c_void_p(16), None, ctypes.c_void_p(16), None)
    assert lib.minih3_time_embed(ctypes.byref(tc), ctypes.byref(mlp), None, None, None, 0.0, 64,
                                 ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 30, None) == m.E_ARG
    assert lib.minih3_time_embed(ctypes.byref(tc), ctypes.byref(mlp), ctypes.c_void_p(16), None, None, 0.0, 64,
                                 ctypes.c_void_p(16), ctypes.c_void_p(16), 10, None) == m.E_WORKSPACE
    cfg = dv.config_for(synth.workload_dims("clip32k"))
    assert lib.minih3_adaln_table_workspace_bytes(ctypes.byref(cfg), 2688, ctypes.byref(n)) == m.OK
    assert n.value >= 64 * 2688 * 2
    p = ctypes.c_void_p(16)
    assert lib.minih3_adaln_table(ctypes.byref(cfg), p, 2688, p, None, p, p, 10, None) == m.E_WORKSPACE
    assert lib.minih3_adaln_table(ctypes.byref(cfg), p, 2680, p, None, p, p, 1 << 30, None) == m.E_UNSUPPORTED
    assert lib.minih3_adaln_table(ctypes.byref(cfg), None, 2688, p, None, p, p, 1 << 30, None) == m.E_ARG


def test_edges_host_side_checks():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libminih3.so not built")
    lib = m.lib()
    cfg = dv.config_for(synth.workload_dims("clip32k"))
    p = ctypes.c_void_p(16)
    e = m._Edges(96, 32, 1e-5, *([p] * 10))
    n = ctypes.c_size_t(0)
    assert lib.minih3_edges_workspace_bytes(ctypes.byref(cfg), ctypes.byref(e), 32768, ctypes.byref(n)) == m.OK
    # validation scratch plus the folded heads (128 x 5376 fp32)
    assert n.value >= 32768 * 4 + 128 * 5376 * 4
    bad = m._Edges(90, 32, 1e-5, *([p] * 10))
    assert lib.minih3_edges_workspace_bytes(ctypes.byref(cfg), ctypes.byref(bad), 32768, ctypes.byref(n)) == \
        m.E_UNSUPPORTED
    L = m._Layout(1, 8, p, p, p, p, 4, p, 2, p, 2)
    assert lib.minih3_embed_inputs(ctypes.byref(cfg), ctypes.byref(L), ctypes.byref(e), p, p, p, p, p, 10, 0,
                                   None) == m.E_WORKSPACE
    assert lib.minih3_output_heads(ctypes.byref(cfg), ctypes.byref(L), ctypes.byref(e), None, p, p, p, 1 << 30, 0,
                                   None) == m.E_ARG
    no_w = m._Edges(96, 32, 1e-5, None, *([p] * 9))
    assert lib.minih3_output_heads(ctypes.byref(cfg), ctypes.byref(L), ctypes.byref(no_w), p, p, p, p, 1 << 30, 0,
                                   None) == m.E_ARG


def test_empty_inputs_are_argument_errors():
    # zero-size sequences and matrices are refused on the host, before any
    # GPU work; a modality with no rows is not an error (the Euler step over
    # zero rows returns at once)
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libminih3.so not built")
    lib = m.lib()
    cfg = dv.config_for(synth.workload_dims("clip32k"))
    p = ctypes.c_void_p(16)
    n = ctypes.c_size_t(0)
    for b, s in ((1, 0), (0, 8), (1, -3)):
        assert lib.minih3_workspace_bytes(ctypes.byref(cfg), b, s, ctypes.byref(n)) == m.E_ARG
        assert lib.minih3_attention_workspace_bytes(ctypes.byref(cfg), b, s, ctypes.byref(n)) == m.E_ARG
        L = m._Layout(b, s, p, p, p, None, 0, None, 0, None, 0)
        bw = (m._BlockWeights * 1)(m._BlockWeights(*[p] * 7))
        assert lib.minih3_block_forward(ctypes.byref(cfg), ctypes.byref(L), bw, 1, p, ctypes.c_void_p(32),
                                        ctypes.c_void_p(64), 1 << 40, 0, None, None) == m.E_ARG
        assert lib.minih3_attention_packed(ctypes.byref(cfg), ctypes.byref(L), p, p, p, ctypes.c_void_p(32), 0.0,
                                           ctypes.c_void_p(64), 1 << 40, 0, None) == m.E_ARG
        assert lib.minih3_adaln_modulate(ctypes.byref(cfg), ctypes.byref(L), p, p, 0, ctypes.c_void_p(32), 0,
                                         None) == m.E_ARG
        assert lib.minih3_qk_norm_rope(ctypes.byref(cfg), ctypes.byref(L), p, p, p, p, p, p, 64, None) == m.E_ARG
    for M, N, K in ((0, 256, 64), (4, 0, 64), (4, 256, 0)):
        assert lib.minih3_linear(0, p, p, ctypes.c_void_p(32), M, N, K, None) == m.E_ARG
        assert lib.minih3_linear_w8a8(p, p, p, p, ctypes.c_void_p(32), M, N, K, None) == m.E_ARG
    assert lib.minih3_rotate_quantize(0, p, 0, 256, p, p, None) == m.E_ARG
    assert lib.minih3_euler_step(None, None, None, 1, 0, 32, None, None, 8, None, None, 8, None) == m.OK
    assert lib.minih3_euler_step(None, None, None, 1, -1, 32, None, None, 8, None, None, 8, None) == m.E_ARG


def test_block_dims_outside_the_kernels_are_refused():
    # an odd head count (QKV width 3 * H * 128 not a multiple of 256), a
    # residual width beyond the AdaLN kernels' row, a head size other than 128
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libminih3.so not built")
    lib = m.lib()
    base = dv.config_for(synth.workload_dims("clip32k"))
    n = ctypes.c_size_t(0)
    assert lib.minih3_workspace_bytes(ctypes.byref(base), 1, 64, ctypes.byref(n)) == m.OK
    for field, value in (("num_heads", 55), ("hidden", 8448), ("head_dim", 64), ("hidden", 5000), ("ffn_dim", 100)):
        bad = m.Config(**{f: getattr(base, f) for f, _ in m.Config._fields_})
        setattr(bad, field, value)
        assert lib.minih3_workspace_bytes(ctypes.byref(bad), 1, 64, ctypes.byref(n)) == m.E_UNSUPPORTED, field
    f32 = m.Config(**{f: getattr(base, f) for f, _ in m.Config._fields_})
    f32.act_dtype = m.F32
    assert lib.minih3_workspace_bytes(ctypes.byref(f32), 1, 64, ctypes.byref(n)) == m.E_UNSUPPORTED  # 5376 > 4096
    f32.hidden = 4096
    assert lib.minih3_workspace_bytes(ctypes.byref(f32), 1, 64, ctypes.byref(n)) == m.OK
