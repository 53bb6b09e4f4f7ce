"""fp64 CPU oracle of the pieces of a denoising step around the blocks: the
unmerged LoRA linear layer and the flow-matching Euler update (TEST
INFRASTRUCTURE ONLY).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. It shares no code with the HIP path.

Sources: page "HyperFlow for MiniMax-H3", header table (a PEFT LoRA of rank
256 and alpha 256 on the attention and feed-forward layers; sampling on a
fixed sigma grid with video shift 12 and audio shift 3) and How it works
(each step hands its endpoints to the embedder); page
"MiniMaxH3Transformer3DModel", `forward` (attention_kwargs may carry a scale
applied to the LoRA layers; the model returns the video and audio
velocities). Readings:
  a. LoRA (PEFT form): y = x W^T + scale * (alpha / rank) * (x A^T) B^T with
     A [rank, in] and B [out, rank]; unmerged, the base weight is untouched;
  b. timestep shift: sigma' = s * sigma / (1 + (s - 1) * sigma);
  c. Euler step of the flow: x_next = x + (sigma_next - sigma_now) * v, with
     the pair (sigma_now, sigma_next) of the row's timestep value.
"""
from __future__ import annotations

import numpy as np


def lora_linear(x, w, a, b, alpha: float, rank: int, scale: float = 1.0) -> np.ndarray:
    """Unmerged LoRA linear layer (reading a)."""
    x = np.asarray(x, np.float64)
    base = x @ np.asarray(w, np.float64).T
    low = (x @ np.asarray(a, np.float64).T) @ np.asarray(b, np.float64).T
    return base + scale * (alpha / rank) * low


def lora_merged_weight(w, a, b, alpha: float, rank: int, scale: float = 1.0) -> np.ndarray:
    """The merged weight W + scale * (alpha / rank) * B A."""
    return np.asarray(w, np.float64) + scale * (alpha / rank) * (np.asarray(b, np.float64) @ np.asarray(a, np.float64))


def shift_sigmas(sigmas, shift: float) -> np.ndarray:
    """Timestep shift of a sigma grid (reading b)."""
    s = np.asarray(sigmas, np.float64)
    return shift * s / (1.0 + (shift - 1.0) * s)


def euler_step(x, v, sigma_now, sigma_next) -> np.ndarray:
    """One Euler step of the flow (reading c); sigmas broadcast per row."""
    x = np.asarray(x, np.float64)
    d = (np.asarray(sigma_next, np.float64) - np.asarray(sigma_now, np.float64))
    return x + d[..., None] * np.asarray(v, np.float64)
