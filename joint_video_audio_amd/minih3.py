"""ctypes binding of libminih3.so (declared in include/minih3.h).

Argument marshalling only: every step of the block runs in the library's
HIP kernels. torch supplies device memory (``tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``). Importing this module
loads nothing; the first call loads the library and raises
``Minih3Error`` if it has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libminih3.so")

BF16, F32 = 0, 1
VALIDATE, ASSUME_PADLESS, PROFILE = 1, 2, 4

OK = 0
E_ARG, E_WORKSPACE, E_UNSUPPORTED, E_SCRATCH = -1, -2, -3, -4
E_LAYOUT_TAG, E_LAYOUT_TVAL, E_LAYOUT_INDEX, E_LAYOUT_PAD, E_NEEDS_MASK = -10, -11, -12, -13, -14
E_HIP = -20

_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn_dim", ctypes.c_int32), ("rope_freq_dim", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("norm_eps", ctypes.c_float), ("qk_norm_eps", ctypes.c_float), ("num_tags", ctypes.c_int32),
                ("num_tvals", ctypes.c_int32), ("tag_text", ctypes.c_int32), ("tag_video", ctypes.c_int32),
                ("tag_audio", ctypes.c_int32), ("act_dtype", ctypes.c_int32)]


class _Layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("token_tags", _P),
                ("timestep_indices", _P), ("position_ids", _P), ("video_indices", _P), ("num_video", ctypes.c_int32),
                ("audio_indices", _P), ("num_audio", ctypes.c_int32), ("text_indices", _P),
                ("num_text", ctypes.c_int32)]


class _BlockWeights(ctypes.Structure):
    _fields_ = [("w_qkv", _P), ("w_out", _P), ("w_gate_up", _P), ("w_down", _P), ("q_norm", _P), ("k_norm", _P),
                ("adaln_table", _P)]


class _BlockWeightsW8A8(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("q_qkv", "s_qkv", "q_out", "s_out", "q_gate_up", "s_gate_up", "q_down", "s_down",
                                  "q_norm", "k_norm", "adaln_table")]


class _StepWeights(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("blocks", _P), ("qblocks", _P), ("edges", _P), ("sigma_now", _P),
                ("sigma_next", _P), ("loras", _P), ("lora_rank", ctypes.c_int32), ("lora_scale", ctypes.c_float)]


class _BlockLora(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("a_qkv", "packed_qkv", "a_out", "packed_out", "a_gate_up", "packed_gate_up",
                                  "a_down", "packed_down")]


TAP_FLOAT = ("adaln1", "q_rot", "k_rot", "v_t", "attn_o", "attn_proj", "x_mid", "adaln2", "ffn_h", "ffn_out")
TAP_INT = ("table_row", "doc_id", "tile_flags", "num_pad")


class _Taps(ctypes.Structure):
    _fields_ = [(n, _P) for n in TAP_FLOAT + TAP_INT + ("block_out",)]


class TimeConfig(ctypes.Structure):
    _fields_ = [("freq_dim", ctypes.c_int32), ("hidden_dim", ctypes.c_int32), ("embed_dim", ctypes.c_int32),
                ("max_period", ctypes.c_float)]


class _TimeMLP(ctypes.Structure):
    _fields_ = [("w1", _P), ("b1", _P), ("w2", _P), ("b2", _P)]


class _TimeMLPLora(ctypes.Structure):
    _fields_ = [("a1", _P), ("packed1", _P), ("a2", _P), ("packed2", _P)]


class _Edges(ctypes.Structure):
    _fields_ = [("video_channels", ctypes.c_int32), ("audio_channels", ctypes.c_int32),
                ("final_norm_eps", ctypes.c_float)] + [(n, _P) for n in (
                    "w_in", "b_in", "w_audio_in", "b_audio_in", "norm_w", "norm_b", "w_out", "b_out", "w_audio_out",
                    "b_audio_out")]


class Minih3Error(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = status_string(status) if _lib_loaded() else str(status)
        super().__init__(f"{what}: {msg} ({status})" if what else f"{msg} ({status})")


_LIB = None


def _lib_loaded() -> bool:
    return _LIB is not None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise Minih3Error(E_HIP, f"{LIB_PATH} is not built (python -m joint_video_audio_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.minih3_status_string.restype = ctypes.c_char_p
        L.minih3_status_string.argtypes = [ctypes.c_int]
        L.minih3_kernel_name.restype = ctypes.c_char_p
        L.minih3_kernel_name.argtypes = [ctypes.c_int32]
        L.minih3_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_attention_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_block_forward.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout),
                                           ctypes.POINTER(_BlockWeights), ctypes.c_int32, _P, _P, _P,
                                           ctypes.c_size_t, ctypes.c_uint32, ctypes.POINTER(_Taps), _P]
        L.minih3_attention_packed.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout), _P, _P, _P, _P,
                                              ctypes.c_float, _P, ctypes.c_size_t, ctypes.c_uint32, _P]
        L.minih3_attention_headmajor_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32,
                                                                 ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_attention_headmajor.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout), _P, _P, _P,
                                                 ctypes.c_int32, _P, ctypes.c_float, _P, ctypes.c_size_t,
                                                 ctypes.c_uint32, _P]
        L.minih3_adaln_modulate.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout), _P, _P, ctypes.c_int32,
                                            _P, ctypes.c_uint32, _P]
        L.minih3_qk_norm_rope.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout), _P, _P, _P, _P, _P, _P,
                                          ctypes.c_int32, _P]
        L.minih3_linear.argtypes = [ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
        L.minih3_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), _I32P, ctypes.c_int32]
        L.minih3_time_embed_workspace_bytes.argtypes = [ctypes.POINTER(TimeConfig), ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_time_embed.argtypes = [ctypes.POINTER(TimeConfig), ctypes.POINTER(_TimeMLP), _P,
                                        ctypes.POINTER(_TimeMLP), _P, ctypes.c_float, ctypes.c_int32, _P, _P,
                                        ctypes.c_size_t, _P]
        L.minih3_time_embed_lora_workspace_bytes.argtypes = [ctypes.POINTER(TimeConfig), ctypes.c_int32,
                                                             ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_time_embed_lora.argtypes = [ctypes.POINTER(TimeConfig), ctypes.POINTER(_TimeMLP),
                                             ctypes.POINTER(_TimeMLPLora), _P, ctypes.POINTER(_TimeMLP),
                                             ctypes.POINTER(_TimeMLPLora), _P, ctypes.c_float, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
        L.minih3_time_embed_lora_workspace_bytes.restype = ctypes.c_int
        L.minih3_time_embed_lora.restype = ctypes.c_int
        L.minih3_adaln_table_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32,
                                                         ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_adaln_table.argtypes = [ctypes.POINTER(Config), _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_size_t,
                                         _P]
        L.minih3_adaln_table_noalloc.argtypes = [ctypes.POINTER(Config), _P, ctypes.c_int32, _P, _P, _P, _P]
        L.minih3_adaln_table_noalloc.restype = ctypes.c_int
        L.minih3_edges_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Edges), ctypes.c_int32,
                                                   ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_embed_inputs.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout), ctypes.POINTER(_Edges), _P,
                                          _P, _P, _P, _P, ctypes.c_size_t, ctypes.c_uint32, _P]
        L.minih3_output_heads.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout), ctypes.POINTER(_Edges), _P,
                                          _P, _P, _P, ctypes.c_size_t, ctypes.c_uint32, _P]
        L.minih3_rotate_quantize.argtypes = [ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
        L.minih3_workspace_bytes_w8a8.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_block_forward_w8a8.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout),
                                                ctypes.POINTER(_BlockWeightsW8A8), ctypes.c_int32, _P, _P, _P,
                                                ctypes.c_size_t, ctypes.c_uint32, ctypes.POINTER(_Taps), _P]
        L.minih3_workspace_bytes_lora.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_block_forward_lora.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout),
                                                ctypes.POINTER(_BlockWeights), ctypes.POINTER(_BlockLora),
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P,
                                                ctypes.c_size_t, ctypes.c_uint32, ctypes.POINTER(_Taps), _P]
        L.minih3_workspace_bytes_lora.restype = ctypes.c_int
        L.minih3_block_forward_lora.restype = ctypes.c_int
        L.minih3_linear_w8a8.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
        L.minih3_lora_pack_weight.argtypes = [ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, _P]
        L.minih3_linear_lora_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_linear_lora.argtypes = [ctypes.c_int32, _P, _P, _P, ctypes.c_float, _P, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P]
        L.minih3_euler_step.argtypes = [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                        ctypes.c_int32, _P, _P, ctypes.c_int32, _P]
        L.minih3_denoise_step_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_StepWeights),
                                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.minih3_denoise_step.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Layout),
                                          ctypes.POINTER(_StepWeights), _P, _P, _P, _P, ctypes.c_size_t,
                                          ctypes.c_uint32, _P]
        for fn in ("minih3_lora_pack_weight", "minih3_linear_lora_workspace_bytes", "minih3_linear_lora",
                   "minih3_euler_step", "minih3_denoise_step_workspace_bytes", "minih3_denoise_step"):
            getattr(L, fn).restype = ctypes.c_int
        for fn in ("minih3_edges_workspace_bytes", "minih3_embed_inputs", "minih3_output_heads",
                   "minih3_rotate_quantize", "minih3_linear_w8a8", "minih3_workspace_bytes_w8a8",
                   "minih3_block_forward_w8a8"):
            getattr(L, fn).restype = ctypes.c_int
        for fn in ("minih3_workspace_bytes", "minih3_attention_workspace_bytes", "minih3_block_forward",
                   "minih3_attention_packed", "minih3_attention_headmajor_workspace_bytes",
                   "minih3_attention_headmajor", "minih3_adaln_modulate", "minih3_qk_norm_rope", "minih3_linear",
                   "minih3_profile_collect", "minih3_time_embed_workspace_bytes", "minih3_time_embed",
                   "minih3_adaln_table_workspace_bytes", "minih3_adaln_table"):
            getattr(L, fn).restype = ctypes.c_int
        _LIB = L
    return _LIB


EXPORTED = ("minih3_workspace_bytes", "minih3_block_forward", "minih3_attention_workspace_bytes",
            "minih3_attention_packed", "minih3_attention_headmajor_workspace_bytes", "minih3_attention_headmajor",
            "minih3_adaln_modulate", "minih3_qk_norm_rope", "minih3_linear",
            "minih3_profile_collect", "minih3_kernel_name", "minih3_status_string",
            "minih3_time_embed_workspace_bytes", "minih3_time_embed", "minih3_time_embed_lora_workspace_bytes",
            "minih3_time_embed_lora", "minih3_adaln_table_workspace_bytes",
            "minih3_adaln_table", "minih3_adaln_table_noalloc", "minih3_edges_workspace_bytes", "minih3_embed_inputs", "minih3_output_heads",
            "minih3_rotate_quantize", "minih3_linear_w8a8", "minih3_workspace_bytes_w8a8",
            "minih3_block_forward_w8a8", "minih3_workspace_bytes_lora", "minih3_block_forward_lora",
            "minih3_lora_pack_weight", "minih3_linear_lora_workspace_bytes",
            "minih3_linear_lora", "minih3_euler_step", "minih3_denoise_step_workspace_bytes",
            "minih3_denoise_step")


def status_string(s: int) -> str:
    return lib().minih3_status_string(int(s)).decode()


def _check(s: int, what: str):
    if s != OK:
        raise Minih3Error(s, what)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _req(t: torch.Tensor, dtype: torch.dtype, name: str, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def act_torch_dtype(cfg: Config) -> torch.dtype:
    return torch.bfloat16 if cfg.act_dtype == BF16 else torch.float32


# --------------------------------------------------------------------------
# layout on the device

class DeviceLayout:
    """int32 device copies of one packed layout (shared by all batch items)."""

    def __init__(self, batch: int, token_tags, timestep_indices, position_ids, video_indices, audio_indices,
                 text_indices, device="cuda"):
        def i32(a):
            t = torch.as_tensor(a)
            return t.to(device=device, dtype=torch.int32).contiguous()

        self.batch = int(batch)
        self.token_tags = i32(token_tags)
        self.timestep_indices = i32(timestep_indices)
        self.position_ids = i32(position_ids).reshape(-1, 3).contiguous()
        self.video_indices = i32(video_indices)
        self.audio_indices = i32(audio_indices)
        self.text_indices = i32(text_indices)
        self.seq_len = int(self.token_tags.numel())
        if self.timestep_indices.numel() != self.seq_len or self.position_ids.shape[0] != self.seq_len:
            raise ValueError("token_tags, timestep_indices and position_ids must describe the same rows")

    @property
    def seq_stride(self) -> int:
        return (self.seq_len + 63) // 64 * 64

    def c(self) -> _Layout:
        def p(t):
            return ctypes.c_void_p(t.data_ptr()) if t.numel() else None

        return _Layout(self.batch, self.seq_len, p(self.token_tags), p(self.timestep_indices), p(self.position_ids),
                       p(self.video_indices), self.video_indices.numel(), p(self.audio_indices),
                       self.audio_indices.numel(), p(self.text_indices), self.text_indices.numel())


class DeviceBlock:
    """Device weights of one block (matrices in act dtype, norms/table fp32)."""

    def __init__(self, w_qkv, w_out, w_gate_up, w_down, q_norm, k_norm, adaln_table):
        self.w_qkv, self.w_out, self.w_gate_up, self.w_down = w_qkv, w_out, w_gate_up, w_down
        self.q_norm, self.k_norm, self.adaln_table = q_norm, k_norm, adaln_table

    def check(self, cfg: Config):
        dt = act_torch_dtype(cfg)
        D, W, F, hd = cfg.hidden, cfg.num_heads * cfg.head_dim, cfg.ffn_dim, cfg.head_dim
        _req(self.w_qkv, dt, "w_qkv", 3 * W * D)
        _req(self.w_out, dt, "w_out", D * W)
        _req(self.w_gate_up, dt, "w_gate_up", 2 * F * D)
        _req(self.w_down, dt, "w_down", D * F)
        _req(self.q_norm, torch.float32, "q_norm", hd)
        _req(self.k_norm, torch.float32, "k_norm", hd)
        _req(self.adaln_table, torch.float32, "adaln_table", cfg.num_tags * cfg.num_tvals * 6 * D)

    def c(self) -> _BlockWeights:
        return _BlockWeights(*(ctypes.c_void_p(t.data_ptr()) for t in (
            self.w_qkv, self.w_out, self.w_gate_up, self.w_down, self.q_norm, self.k_norm, self.adaln_table)))


# --------------------------------------------------------------------------
# entry points

def workspace_bytes(cfg: Config, batch: int, seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().minih3_workspace_bytes(ctypes.byref(cfg), batch, seq_len, ctypes.byref(n)), "workspace_bytes")
    return int(n.value)


def attention_workspace_bytes(cfg: Config, batch: int, seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().minih3_attention_workspace_bytes(ctypes.byref(cfg), batch, seq_len, ctypes.byref(n)),
           "attention_workspace_bytes")
    return int(n.value)


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def block_forward(cfg: Config, layout: DeviceLayout, blocks: Sequence[DeviceBlock], x: torch.Tensor,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, flags: int = 0,
                  taps: Optional[dict] = None) -> torch.Tensor:
    """x [B, S, D] -> out [B, S, D] through len(blocks) chained blocks."""
    dt = act_torch_dtype(cfg)
    B, S, D = layout.batch, layout.seq_len, cfg.hidden
    _req(x, dt, "x", B * S * D)
    for b in blocks:
        b.check(cfg)
    if out is None:
        out = torch.empty_like(x)
    _req(out, dt, "out", B * S * D)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(cfg, B, S), x.device)
    arr = (_BlockWeights * len(blocks))(*[b.c() for b in blocks])
    ct = None
    if taps:
        ct = _Taps(**{k: (ctypes.c_void_p(v.data_ptr()) if v is not None else None) for k, v in taps.items()})
    L = layout.c()
    s = lib().minih3_block_forward(ctypes.byref(cfg), ctypes.byref(L), arr, len(blocks), _ptr(x), _ptr(out),
                                   _ptr(workspace), workspace.numel(), flags,
                                   ctypes.byref(ct) if ct is not None else None, _stream())
    _check(s, "block_forward")
    return out


def attention_packed(cfg: Config, layout: DeviceLayout, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0, flags: int = 0,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q, k, v [B, S, H, hd] (q, k after norm and rotary) -> out [B, S, H*hd]."""
    dt = act_torch_dtype(cfg)
    B, H, hd, S = layout.batch, cfg.num_heads, cfg.head_dim, layout.seq_len
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, dt, n, B * S * H * hd)
    if out is None:
        out = torch.empty(B, S, H * hd, dtype=dt, device=q.device)
    _req(out, dt, "out", B * S * H * hd)
    if workspace is None:
        workspace = alloc_workspace(attention_workspace_bytes(cfg, B, S), q.device)
    L = layout.c()
    s = lib().minih3_attention_packed(ctypes.byref(cfg), ctypes.byref(L), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                      float(softmax_scale), _ptr(workspace), workspace.numel(), flags, _stream())
    _check(s, "attention_packed")
    return out


def attention_headmajor_workspace_bytes(cfg: Config, batch: int, seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().minih3_attention_headmajor_workspace_bytes(ctypes.byref(cfg), batch, seq_len, ctypes.byref(n)),
           "attention_headmajor_workspace_bytes")
    return int(n.value)


def attention_headmajor(cfg: Config, layout: DeviceLayout, q: torch.Tensor, k: torch.Tensor, v_t: torch.Tensor,
                        out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0, flags: int = 0,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q, k [B, H, stride, hd], v_t [B, H, hd, stride] -> out [B, S, H*hd]."""
    dt = act_torch_dtype(cfg)
    B, H, hd, S = layout.batch, cfg.num_heads, cfg.head_dim, layout.seq_len
    stride = q.shape[2]
    for t, n in ((q, "q"), (k, "k"), (v_t, "v_t")):
        _req(t, dt, n, B * H * stride * hd)
    if out is None:
        out = torch.empty(B, S, H * hd, dtype=dt, device=q.device)
    _req(out, dt, "out", B * S * H * hd)
    if workspace is None:
        workspace = alloc_workspace(attention_headmajor_workspace_bytes(cfg, B, S), q.device)
    L = layout.c()
    s = lib().minih3_attention_headmajor(ctypes.byref(cfg), ctypes.byref(L), _ptr(q), _ptr(k), _ptr(v_t), stride,
                                         _ptr(out), float(softmax_scale), _ptr(workspace), workspace.numel(), flags,
                                         _stream())
    _check(s, "attention_headmajor")
    return out


def adaln_modulate(cfg: Config, layout: DeviceLayout, x: torch.Tensor, adaln_table: torch.Tensor, which: int,
                   y: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    dt = act_torch_dtype(cfg)
    B, S, D = layout.batch, layout.seq_len, cfg.hidden
    _req(x, dt, "x", B * S * D)
    _req(adaln_table, torch.float32, "adaln_table", cfg.num_tags * cfg.num_tvals * 6 * D)
    if y is None:
        y = torch.empty_like(x)
    _req(y, dt, "y", B * S * D)
    L = layout.c()
    _check(lib().minih3_adaln_modulate(ctypes.byref(cfg), ctypes.byref(L), _ptr(x), _ptr(adaln_table), which,
                                       _ptr(y), flags, _stream()), "adaln_modulate")
    return y


def qk_norm_rope(cfg: Config, layout: DeviceLayout, qkv: torch.Tensor, q_norm: torch.Tensor, k_norm: torch.Tensor):
    """qkv [B, S, 3W] -> (q, k [B, H, stride, hd], v_t [B, H, hd, stride])."""
    dt = act_torch_dtype(cfg)
    B, S, H, hd = layout.batch, layout.seq_len, cfg.num_heads, cfg.head_dim
    _req(qkv, dt, "qkv", B * S * 3 * H * hd)
    _req(q_norm, torch.float32, "q_norm", hd)
    _req(k_norm, torch.float32, "k_norm", hd)
    st = layout.seq_stride
    q = torch.empty(B, H, st, hd, dtype=dt, device=qkv.device)
    k = torch.empty_like(q)
    vt = torch.empty(B, H, hd, st, dtype=dt, device=qkv.device)
    L = layout.c()
    _check(lib().minih3_qk_norm_rope(ctypes.byref(cfg), ctypes.byref(L), _ptr(qkv), _ptr(q_norm), _ptr(k_norm),
                                     _ptr(q), _ptr(k), _ptr(vt), st, _stream()), "qk_norm_rope")
    return q, k, vt


def linear(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[M, N] = a[M, K] . w[N, K]^T (bf16 or fp32)."""
    if a.dtype == torch.bfloat16:
        dtc = BF16
    elif a.dtype == torch.float32:
        dtc = F32
    else:
        raise ValueError("a must be bf16 or fp32")
    M, K = a.shape
    N = w.shape[0]
    _req(a, a.dtype, "a")
    _req(w, a.dtype, "w", N * K)
    if out is None:
        out = torch.empty(M, N, dtype=a.dtype, device=a.device)
    _req(out, a.dtype, "out", M * N)
    _check(lib().minih3_linear(dtc, _ptr(a), _ptr(w), _ptr(out), M, N, K, _stream()), "linear")
    return out


class DeviceTimeMLP:
    """fp32 device weights of one timestep MLP (w1 [hidden, freq], w2 [embed, hidden])."""

    def __init__(self, w1, b1, w2, b2):
        self.w1, self.b1, self.w2, self.b2 = w1, b1, w2, b2

    def check(self, tc: TimeConfig):
        _req(self.w1, torch.float32, "w1", tc.hidden_dim * tc.freq_dim)
        _req(self.w2, torch.float32, "w2", tc.embed_dim * tc.hidden_dim)
        if self.b1 is not None:
            _req(self.b1, torch.float32, "b1", tc.hidden_dim)
        if self.b2 is not None:
            _req(self.b2, torch.float32, "b2", tc.embed_dim)

    def c(self) -> _TimeMLP:
        return _TimeMLP(*(_ptr(t) for t in (self.w1, self.b1, self.w2, self.b2)))


def time_embed_workspace_bytes(tc: TimeConfig, num_tvals: int) -> int:
    nb = ctypes.c_size_t(0)
    _check(lib().minih3_time_embed_workspace_bytes(ctypes.byref(tc), num_tvals, ctypes.byref(nb)),
           "time_embed_workspace_bytes")
    return int(nb.value)


def time_embed(tc: TimeConfig, base: DeviceTimeMLP, t: torch.Tensor, endpoint: Optional[DeviceTimeMLP] = None,
               r: Optional[torch.Tensor] = None, gate: float = 0.0, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """t [n] fp32 -> time embeddings [n, embed_dim] fp32 (two-time blend with an endpoint MLP)."""
    n = t.numel()
    _req(t, torch.float32, "t", n)
    base.check(tc)
    if endpoint is not None:
        endpoint.check(tc)
    if r is not None:
        _req(r, torch.float32, "r", n)
    if out is None:
        out = torch.empty(n, tc.embed_dim, dtype=torch.float32, device=t.device)
    _req(out, torch.float32, "out", n * tc.embed_dim)
    ws = workspace if workspace is not None else alloc_workspace(time_embed_workspace_bytes(tc, n), t.device)
    cb = base.c()
    ce = endpoint.c() if endpoint is not None else None
    _check(lib().minih3_time_embed(ctypes.byref(tc), ctypes.byref(cb), _ptr(t),
                                   ctypes.byref(ce) if ce is not None else None, _ptr(r), float(gate), n, _ptr(out),
                                   _ptr(ws), ws.numel(), _stream()), "time_embed")
    return out


class DeviceTimeMLPLora:
    """Unmerged adapter of one timestep MLP (fp32): a1 [rank, freq], packed1 = [W1 | B1], a2 [rank, hidden],
    packed2 = [W2 | B2]."""

    def __init__(self, a1, packed1, a2, packed2):
        self.a1, self.packed1, self.a2, self.packed2 = a1, packed1, a2, packed2
        self.rank = int(a1.shape[0])

    @classmethod
    def from_mlp(cls, mlp: DeviceTimeMLP, a1, b1, a2, b2) -> "DeviceTimeMLPLora":
        return cls(a1, lora_pack_weight(mlp.w1, b1), a2, lora_pack_weight(mlp.w2, b2))

    def check(self, tc: TimeConfig):
        r = self.rank
        _req(self.a1, torch.float32, "a1", r * tc.freq_dim)
        _req(self.packed1, torch.float32, "packed1", tc.hidden_dim * (tc.freq_dim + r))
        _req(self.a2, torch.float32, "a2", r * tc.hidden_dim)
        _req(self.packed2, torch.float32, "packed2", tc.embed_dim * (tc.hidden_dim + r))

    def c(self) -> _TimeMLPLora:
        return _TimeMLPLora(*(_ptr(t) for t in (self.a1, self.packed1, self.a2, self.packed2)))


def time_embed_lora(tc: TimeConfig, base: DeviceTimeMLP, base_lora: DeviceTimeMLPLora, t: torch.Tensor,
                    lora_scale: float, endpoint: Optional[DeviceTimeMLP] = None,
                    endpoint_lora: Optional[DeviceTimeMLPLora] = None, r: Optional[torch.Tensor] = None,
                    gate: float = 0.0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """time_embed with unmerged adapters on the timestep MLPs (lora_scale = scale * alpha / rank)."""
    n = t.numel()
    _req(t, torch.float32, "t", n)
    base_lora.check(tc)
    if endpoint is not None:
        if endpoint_lora is None:
            raise ValueError("an endpoint MLP needs its adapter")
        endpoint_lora.check(tc)
        if endpoint_lora.rank != base_lora.rank:
            raise ValueError("the two adapters share a rank")
    if r is not None:
        _req(r, torch.float32, "r", n)
    if out is None:
        out = torch.empty(n, tc.embed_dim, dtype=torch.float32, device=t.device)
    _req(out, torch.float32, "out", n * tc.embed_dim)
    rank = base_lora.rank
    if workspace is None:
        nb = ctypes.c_size_t(0)
        _check(lib().minih3_time_embed_lora_workspace_bytes(ctypes.byref(tc), n, rank, ctypes.byref(nb)),
               "time_embed_lora_workspace_bytes")
        workspace = alloc_workspace(int(nb.value), t.device)
    cb, cl = base.c(), base_lora.c()
    ce = endpoint.c() if endpoint is not None else None
    cel = endpoint_lora.c() if endpoint is not None else None
    _check(lib().minih3_time_embed_lora(ctypes.byref(tc), ctypes.byref(cb), ctypes.byref(cl), _ptr(t),
                                        ctypes.byref(ce) if ce is not None else None,
                                        ctypes.byref(cel) if cel is not None else None, _ptr(r), float(gate), n,
                                        rank, float(lora_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                        _stream()), "time_embed_lora")
    return out


def adaln_table_workspace_bytes(cfg: Config, embed_dim: int) -> int:
    nb = ctypes.c_size_t(0)
    _check(lib().minih3_adaln_table_workspace_bytes(ctypes.byref(cfg), embed_dim, ctypes.byref(nb)),
           "adaln_table_workspace_bytes")
    return int(nb.value)


def adaln_table(cfg: Config, emb: torch.Tensor, w_proj: torch.Tensor, b_proj: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """emb [num_tvals, E] fp32, w_proj [tags, 6D, E] act -> table [tags, num_tvals, 6, D] fp32."""
    dt = act_torch_dtype(cfg)
    T, V, D = cfg.num_tags, cfg.num_tvals, cfg.hidden
    E = emb.shape[-1]
    _req(emb, torch.float32, "emb", V * E)
    _req(w_proj, dt, "w_proj", T * 6 * D * E)
    if b_proj is not None:
        _req(b_proj, dt, "b_proj", T * 6 * D)
    if out is None:
        out = torch.empty(T, V, 6, D, dtype=torch.float32, device=emb.device)
    _req(out, torch.float32, "table", T * V * 6 * D)
    if workspace is None:
        workspace = alloc_workspace(adaln_table_workspace_bytes(cfg, E), emb.device)
    _check(lib().minih3_adaln_table(ctypes.byref(cfg), _ptr(emb), E, _ptr(w_proj), _ptr(b_proj), _ptr(out),
                                    _ptr(workspace), workspace.numel(), _stream()), "adaln_table")
    return out


def adaln_table_noalloc(cfg: Config, emb: torch.Tensor, w_proj: torch.Tensor, out: torch.Tensor,
                        b_proj: Optional[torch.Tensor] = None) -> torch.Tensor:
    """adaln_table into a caller-provided `out` with no workspace: the library
    uses its fixed per-device scratch (see minih3_adaln_table_noalloc)."""
    dt = act_torch_dtype(cfg)
    T, V, D = cfg.num_tags, cfg.num_tvals, cfg.hidden
    E = emb.shape[-1]
    _req(emb, torch.float32, "emb", V * E)
    _req(w_proj, dt, "w_proj", T * 6 * D * E)
    if b_proj is not None:
        _req(b_proj, dt, "b_proj", T * 6 * D)
    _req(out, torch.float32, "table", T * V * 6 * D)
    _check(lib().minih3_adaln_table_noalloc(ctypes.byref(cfg), _ptr(emb), E, _ptr(w_proj), _ptr(b_proj), _ptr(out),
                                            _stream()), "adaln_table_noalloc")
    return out


class DeviceEdges:
    """fp32 device weights of the model edges (proj_in, audio_proj_in, norm_out,
    proj_out, audio_proj_out)."""

    NAMES = ("w_in", "b_in", "w_audio_in", "b_audio_in", "norm_w", "norm_b", "w_out", "b_out", "w_audio_out",
             "b_audio_out")

    def __init__(self, video_channels: int, audio_channels: int, final_norm_eps: float, **tensors):
        self.video_channels, self.audio_channels = int(video_channels), int(audio_channels)
        self.final_norm_eps = float(final_norm_eps)
        self.t = {n: tensors.get(n) for n in self.NAMES}

    def check(self, cfg: Config):
        D, Cv, Ca = cfg.hidden, self.video_channels, self.audio_channels
        shapes = dict(w_in=D * Cv, b_in=D, w_audio_in=D * Ca, b_audio_in=D, norm_w=D, norm_b=D, w_out=Cv * D,
                      b_out=Cv, w_audio_out=Ca * D, b_audio_out=Ca)
        for n, k in shapes.items():
            if self.t[n] is None and n in ("b_out", "b_audio_out"):
                continue
            _req(self.t[n], torch.float32, n, k)

    def c(self) -> _Edges:
        return _Edges(self.video_channels, self.audio_channels, self.final_norm_eps,
                      *(_ptr(self.t[n]) for n in self.NAMES))


def edges_workspace_bytes(cfg: Config, edges: DeviceEdges, seq_len: int) -> int:
    nb = ctypes.c_size_t(0)
    ce = edges.c()
    _check(lib().minih3_edges_workspace_bytes(ctypes.byref(cfg), ctypes.byref(ce), seq_len, ctypes.byref(nb)),
           "edges_workspace_bytes")
    return int(nb.value)


def embed_inputs(cfg: Config, layout: DeviceLayout, edges: DeviceEdges, video: torch.Tensor, audio: torch.Tensor,
                 text: torch.Tensor, x: Optional[torch.Tensor] = None, flags: int = 0,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """video [B, n_video, Cv] fp32, audio [B, n_audio, Ca] fp32, text [B, n_text, D] act -> x [B, S, D] act."""
    dt = act_torch_dtype(cfg)
    B, S, D = layout.batch, layout.seq_len, cfg.hidden
    edges.check(cfg)
    _req(video, torch.float32, "video", B * layout.video_indices.numel() * edges.video_channels)
    _req(audio, torch.float32, "audio", B * layout.audio_indices.numel() * edges.audio_channels)
    _req(text, dt, "text", B * layout.text_indices.numel() * D)
    if x is None:
        x = torch.empty(B, S, D, dtype=dt, device=video.device)
    _req(x, dt, "x", B * S * D)
    if workspace is None:
        workspace = alloc_workspace(edges_workspace_bytes(cfg, edges, S), video.device)
    L, ce = layout.c(), edges.c()
    _check(lib().minih3_embed_inputs(ctypes.byref(cfg), ctypes.byref(L), ctypes.byref(ce), _ptr(video), _ptr(audio),
                                     _ptr(text), _ptr(x), _ptr(workspace), workspace.numel(), flags, _stream()),
           "embed_inputs")
    return x


def output_heads(cfg: Config, layout: DeviceLayout, edges: DeviceEdges, x: torch.Tensor, flags: int = 0,
                 workspace: Optional[torch.Tensor] = None):
    """x [B, S, D] act -> (video velocity [B, n_video, Cv], audio velocity [B, n_audio, Ca]) fp32."""
    dt = act_torch_dtype(cfg)
    B, S, D = layout.batch, layout.seq_len, cfg.hidden
    edges.check(cfg)
    _req(x, dt, "x", B * S * D)
    v = torch.empty(B, layout.video_indices.numel(), edges.video_channels, dtype=torch.float32, device=x.device)
    a = torch.empty(B, layout.audio_indices.numel(), edges.audio_channels, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(edges_workspace_bytes(cfg, edges, S), x.device)
    L, ce = layout.c(), edges.c()
    _check(lib().minih3_output_heads(ctypes.byref(cfg), ctypes.byref(L), ctypes.byref(ce), _ptr(x), _ptr(v), _ptr(a),
                                     _ptr(workspace), workspace.numel(), flags, _stream()), "output_heads")
    return v, a


def rotate_quantize(x: torch.Tensor):
    """Rows of x [M, K] (bf16 or fp32) -> (int8 codes [M, K], fp32 scales [M]) after the blockwise
    Hadamard rotation."""
    if x.dtype == torch.bfloat16:
        dtc = BF16
    elif x.dtype == torch.float32:
        dtc = F32
    else:
        raise ValueError("x must be bf16 or fp32")
    M, K = x.shape
    _req(x, x.dtype, "x")
    q = torch.empty(M, K, dtype=torch.int8, device=x.device)
    sc = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().minih3_rotate_quantize(dtc, _ptr(x), M, K, _ptr(q), _ptr(sc), _stream()), "rotate_quantize")
    return q, sc


def linear_w8a8(qa: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 out[M, N] = (qa . qw^T) * sa[m] * sw[n] from int8 codes and fp32 row scales."""
    M, K = qa.shape
    N = qw.shape[0]
    _req(qa, torch.int8, "qa")
    _req(qw, torch.int8, "qw", N * K)
    _req(sa, torch.float32, "sa", M)
    _req(sw, torch.float32, "sw", N)
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=qa.device)
    _req(out, torch.bfloat16, "out", M * N)
    _check(lib().minih3_linear_w8a8(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(out), M, N, K, _stream()),
           "linear_w8a8")
    return out


class DeviceBlockW8A8:
    """Weights of one block for the rotated W8A8 forward: int8 codes and fp32
    row scales of the four matrices (from rotate_quantize), norms and table."""

    NAMES = ("qkv", "out", "gate_up", "down")

    def __init__(self, codes: dict, scales: dict, q_norm, k_norm, adaln_table):
        self.codes, self.scales = codes, scales
        self.q_norm, self.k_norm, self.adaln_table = q_norm, k_norm, adaln_table

    @classmethod
    def from_block(cls, b: DeviceBlock) -> "DeviceBlockW8A8":
        codes, scales = {}, {}
        for n, w in zip(cls.NAMES, (b.w_qkv, b.w_out, b.w_gate_up, b.w_down)):
            codes[n], scales[n] = rotate_quantize(w)
        return cls(codes, scales, b.q_norm, b.k_norm, b.adaln_table)

    def c(self) -> _BlockWeightsW8A8:
        ptrs = []
        for n in self.NAMES:
            ptrs += [_ptr(self.codes[n]), _ptr(self.scales[n])]
        return _BlockWeightsW8A8(*ptrs, _ptr(self.q_norm), _ptr(self.k_norm), _ptr(self.adaln_table))


class DeviceBlockLora:
    """Unmerged adapter of one block: per projection the A matrix [rank, K]
    and the packed [W | B] [N, K + rank] (act dtype)."""

    NAMES = ("qkv", "out", "gate_up", "down")

    def __init__(self, a: dict, packed: dict, rank: int):
        self.a, self.packed, self.rank = a, packed, int(rank)

    @classmethod
    def from_block(cls, b: DeviceBlock, a: dict, bmat: dict) -> "DeviceBlockLora":
        """a[name] [rank, K] and bmat[name] [N, rank] for the four projections of b."""
        packed = {}
        for n, w in zip(cls.NAMES, (b.w_qkv, b.w_out, b.w_gate_up, b.w_down)):
            packed[n] = lora_pack_weight(w, bmat[n])
        return cls({n: a[n] for n in cls.NAMES}, packed, a["qkv"].shape[0])

    def check(self, cfg: Config):
        dt = act_torch_dtype(cfg)
        D, W, F = cfg.hidden, cfg.num_heads * cfg.head_dim, cfg.ffn_dim
        shapes = {"qkv": (3 * W, D), "out": (D, W), "gate_up": (2 * F, D), "down": (D, F)}
        for n, (N, K) in shapes.items():
            _req(self.a[n], dt, f"lora a_{n}", self.rank * K)
            _req(self.packed[n], dt, f"lora packed_{n}", N * (K + self.rank))

    def c(self) -> _BlockLora:
        ptrs = []
        for n in self.NAMES:
            ptrs += [_ptr(self.a[n]), _ptr(self.packed[n])]
        return _BlockLora(*ptrs)


def workspace_bytes_lora(cfg: Config, batch: int, seq_len: int, rank: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().minih3_workspace_bytes_lora(ctypes.byref(cfg), batch, seq_len, rank, ctypes.byref(n)),
           "workspace_bytes_lora")
    return int(n.value)


def block_forward_lora(cfg: Config, layout: DeviceLayout, blocks: Sequence[DeviceBlock],
                       loras: Sequence[DeviceBlockLora], x: torch.Tensor, lora_scale: float,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, flags: int = 0,
                       taps: Optional[dict] = None) -> torch.Tensor:
    """block_forward with the unmerged adapter loras[i] on every projection of blocks[i];
    lora_scale = scale * alpha / rank."""
    dt = act_torch_dtype(cfg)
    B, S, D = layout.batch, layout.seq_len, cfg.hidden
    _req(x, dt, "x", B * S * D)
    if len(loras) != len(blocks):
        raise ValueError("one adapter per block")
    rank = loras[0].rank
    for lb in loras:
        lb.check(cfg)
        if lb.rank != rank:
            raise ValueError("adapters of one call share a rank")
    if out is None:
        out = torch.empty_like(x)
    _req(out, dt, "out", B * S * D)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes_lora(cfg, B, S, rank), x.device)
    arr = (_BlockWeights * len(blocks))(*[b.c() for b in blocks])
    larr = (_BlockLora * len(loras))(*[lb.c() for lb in loras])
    ct = None
    if taps:
        ct = _Taps(**{k: (ctypes.c_void_p(v.data_ptr()) if v is not None else None) for k, v in taps.items()})
    L = layout.c()
    s = lib().minih3_block_forward_lora(ctypes.byref(cfg), ctypes.byref(L), arr, larr, len(blocks), rank,
                                        float(lora_scale), _ptr(x), _ptr(out), _ptr(workspace), workspace.numel(),
                                        flags, ctypes.byref(ct) if ct is not None else None, _stream())
    _check(s, "block_forward_lora")
    return out


def workspace_bytes_w8a8(cfg: Config, batch: int, seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().minih3_workspace_bytes_w8a8(ctypes.byref(cfg), batch, seq_len, ctypes.byref(n)),
           "workspace_bytes_w8a8")
    return int(n.value)


def block_forward_w8a8(cfg: Config, layout: DeviceLayout, blocks: Sequence[DeviceBlockW8A8], x: torch.Tensor,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, flags: int = 0,
                       taps: Optional[dict] = None) -> torch.Tensor:
    """x [B, S, D] bf16 -> out [B, S, D] through the blocks with rotated W8A8 projections."""
    B, S, D = layout.batch, layout.seq_len, cfg.hidden
    _req(x, torch.bfloat16, "x", B * S * D)
    if out is None:
        out = torch.empty_like(x)
    _req(out, torch.bfloat16, "out", B * S * D)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes_w8a8(cfg, B, S), x.device)
    arr = (_BlockWeightsW8A8 * len(blocks))(*[b.c() for b in blocks])
    ct = None
    if taps:
        ct = _Taps(**{k: (ctypes.c_void_p(v.data_ptr()) if v is not None else None) for k, v in taps.items()})
    L = layout.c()
    s = lib().minih3_block_forward_w8a8(ctypes.byref(cfg), ctypes.byref(L), arr, len(blocks), _ptr(x), _ptr(out),
                                        _ptr(workspace), workspace.numel(), flags,
                                        ctypes.byref(ct) if ct is not None else None, _stream())
    _check(s, "block_forward_w8a8")
    return out


def _dtc(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError("bf16 or fp32 expected")


def lora_pack_weight(w: torch.Tensor, lora_b: torch.Tensor) -> torch.Tensor:
    """[W | B]: w [N, K], lora_b [N, rank] -> [N, K + rank] (same dtype)."""
    N, K = w.shape
    r = lora_b.shape[1]
    _req(w, w.dtype, "w")
    _req(lora_b, w.dtype, "lora_b", N * r)
    out = torch.empty(N, K + r, dtype=w.dtype, device=w.device)
    _check(lib().minih3_lora_pack_weight(_dtc(w), _ptr(w), _ptr(lora_b), _ptr(out), N, K, r, _stream()),
           "lora_pack_weight")
    return out


def linear_lora(a: torch.Tensor, lora_a: torch.Tensor, packed: torch.Tensor, lora_scale: float,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[M, N] = a W^T + lora_scale (a A^T) B^T with packed = [W | B] (unmerged LoRA)."""
    M, K = a.shape
    r = lora_a.shape[0]
    N = packed.shape[0]
    dt = a.dtype
    _req(a, dt, "a")
    _req(lora_a, dt, "lora_a", r * K)
    _req(packed, dt, "packed", N * (K + r))
    if out is None:
        out = torch.empty(M, N, dtype=dt, device=a.device)
    _req(out, dt, "out", M * N)
    if workspace is None:
        nb = ctypes.c_size_t(0)
        _check(lib().minih3_linear_lora_workspace_bytes(_dtc(a), M, K, r, ctypes.byref(nb)), "linear_lora")
        workspace = alloc_workspace(int(nb.value), a.device)
    _check(lib().minih3_linear_lora(_dtc(a), _ptr(a), _ptr(lora_a), _ptr(packed), float(lora_scale), _ptr(out), M, N,
                                    K, r, _ptr(workspace), workspace.numel(), _stream()), "linear_lora")
    return out


def euler_step(x: torch.Tensor, velocity: torch.Tensor, indices: torch.Tensor, timestep_indices: torch.Tensor,
               sigma_now: torch.Tensor, sigma_next: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x, velocity [B, n, C] fp32 (rows in the order of indices) -> x + (sigma_next - sigma_now)[row] * velocity."""
    B, n, C = x.shape
    _req(x, torch.float32, "x")
    _req(velocity, torch.float32, "velocity", B * n * C)
    _req(indices, torch.int32, "indices", n)
    _req(timestep_indices, torch.int32, "timestep_indices")
    _req(sigma_now, torch.float32, "sigma_now")
    _req(sigma_next, torch.float32, "sigma_next", sigma_now.numel())
    if out is None:
        out = torch.empty_like(x)
    _req(out, torch.float32, "out", B * n * C)
    _check(lib().minih3_euler_step(_ptr(x), _ptr(velocity), _ptr(out), B, n, C, _ptr(indices),
                                   _ptr(timestep_indices), timestep_indices.numel(), _ptr(sigma_now),
                                   _ptr(sigma_next), sigma_now.numel(), _stream()), "euler_step")
    return out


def denoise_step(cfg: Config, layout: DeviceLayout, blocks, edges: DeviceEdges, sigma_now: torch.Tensor,
                 sigma_next: torch.Tensor, video: torch.Tensor, audio: torch.Tensor, text: torch.Tensor,
                 flags: int = 0, workspace: Optional[torch.Tensor] = None,
                 loras: Optional[Sequence["DeviceBlockLora"]] = None, lora_scale: float = 1.0):
    """One denoising step: video [B, n_video, Cv] and audio [B, n_audio, Ca] fp32 latents are updated in place
    (input projections, the block chain -- DeviceBlock or DeviceBlockW8A8 list, with unmerged adapters on the
    DeviceBlock chain when loras is given (lora_scale = scale * alpha / rank) --, heads, Euler update)."""
    B, S = layout.batch, layout.seq_len
    nv, na = layout.video_indices.numel(), layout.audio_indices.numel()
    edges.check(cfg)
    _req(video, torch.float32, "video", B * nv * edges.video_channels)
    _req(audio, torch.float32, "audio", B * na * edges.audio_channels)
    _req(text, act_torch_dtype(cfg), "text", B * layout.text_indices.numel() * cfg.hidden)
    _req(sigma_now, torch.float32, "sigma_now", cfg.num_tvals)
    _req(sigma_next, torch.float32, "sigma_next", cfg.num_tvals)
    w8 = isinstance(blocks[0], DeviceBlockW8A8)
    if w8:
        arr = (_BlockWeightsW8A8 * len(blocks))(*[b.c() for b in blocks])
    else:
        for b in blocks:
            b.check(cfg)
        arr = (_BlockWeights * len(blocks))(*[b.c() for b in blocks])
    ce = edges.c()
    larr, rank = None, 0
    if loras is not None:
        if w8 or len(loras) != len(blocks):
            raise ValueError("adapters go with the bf16 / fp32 block chain, one per block")
        for lb in loras:
            lb.check(cfg)
        rank = loras[0].rank
        larr = (_BlockLora * len(loras))(*[lb.c() for lb in loras])
    sw = _StepWeights(len(blocks), None if w8 else ctypes.cast(arr, _P), ctypes.cast(arr, _P) if w8 else None,
                      ctypes.cast(ctypes.pointer(ce), _P), _ptr(sigma_now), _ptr(sigma_next),
                      ctypes.cast(larr, _P) if larr is not None else None, rank, float(lora_scale))
    if workspace is None:
        nb = ctypes.c_size_t(0)
        _check(lib().minih3_denoise_step_workspace_bytes(ctypes.byref(cfg), ctypes.byref(sw), B, S, nv, na,
                                                         ctypes.byref(nb)), "denoise_step_workspace_bytes")
        workspace = alloc_workspace(int(nb.value), video.device)
    L = layout.c()
    _check(lib().minih3_denoise_step(ctypes.byref(cfg), ctypes.byref(L), ctypes.byref(sw), _ptr(video), _ptr(audio),
                                     _ptr(text), _ptr(workspace), workspace.numel(), flags, _stream()),
           "denoise_step")
    return video, audio


def profile_collect() -> dict:
    n = 16
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    k = lib().minih3_profile_collect(ms, cnt, n)
    res = {}
    for i in range(k):
        name = lib().minih3_kernel_name(i).decode()
        res[name] = (float(ms[i]), int(cnt[i]))
    return res
