"""Write the expected values of the full-size parity tests.

    python tests/golden/make_golden.py [case ...]

A case is a full-width workload, a seed and a gate recipe (see CASES). For
each case this draws the synthetic inputs with joint_video_audio_amd.synth,
runs the fp64 oracle (oracle/) and stores, as float32, the values of a fixed
sample of packed rows:

  single-block workloads: the block output and the fp32 residual stream
  after the attention's gated add (x_mid) on N_SAMPLE rows; the attention
  output, the output projection, the SwiGLU output and the down projection
  on the first N_TAP of those rows (tap_rows);
  the four-block chain: the chain output and the first block's output on
  N_SAMPLE rows.

The rows cover every run of equal tags (text, conditioning, audio, target
video, padding: first, last and middle row, plus random rows in proportion
to the run's length), the edges of the 256-row projection tiles and 64-row
attention tiles, and the ragged tail. float32 rounding (2^-24 relative) is
negligible against the float bar of the tests. Nothing here touches the
HIP path.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import block as ob  # noqa: E402
from joint_video_audio_amd import synth  # noqa: E402

N_SAMPLE = 256
N_TAP = 64

# (workload, seed, gate mean): the zero-mean gate recipe at seed 0 for every
# full-width workload, the four-block chain also at seeds 1 and 2 (whose
# padding counts differ), and the clip-scale block with gates ~ N(1, 0.1).
CASES = {
    "padless8k_seed0": ("padless8k", 0, 0.0),
    "padded16k_seed0": ("padded16k", 0, 0.0),
    "clip32k_seed0": ("clip32k", 0, 0.0),
    "clip32k_unitgates_seed0": ("clip32k", 0, 1.0),
    "chain4x24k_seed0": ("chain4x24k", 0, 0.0),
    "chain4x24k_seed1": ("chain4x24k", 1, 0.0),
    "chain4x24k_seed2": ("chain4x24k", 2, 0.0),
}


def tag_runs(tags: np.ndarray):
    """(start, end) of every maximal run of equal tags."""
    cut = np.flatnonzero(np.diff(tags)) + 1
    starts = np.concatenate([[0], cut])
    ends = np.concatenate([cut, [tags.shape[0]]])
    return [(int(a), int(b)) for a, b in zip(starts, ends)]


def sample_rows(layout, n: int = N_SAMPLE, n_tap: int = N_TAP):
    """(rows, tap_rows): n sorted distinct rows and the n_tap of them that
    come first in priority order (run ends and middles, tile edges, tail)."""
    S = layout.seq_len
    runs = tag_runs(np.asarray(layout.token_tags))
    pri = []
    for a, b in runs:
        pri += [a, b - 1, (a + b) // 2]
    for e in (64, 256, 512):
        pri += [e - 1, e]
    last256, last64 = (S - 1) // 256 * 256, (S - 1) // 64 * 64
    pri += [S - 1, S - 2, last256, last256 - 1, last64, last64 - 1, S // 2]
    rng = np.random.default_rng(1234)
    for a, b in runs:  # a few random rows of every run, short runs included
        pri += [int(r) for r in rng.integers(a, b, size=4)]
    seen, order = set(), []
    for r in pri:
        if 0 <= r < S and r not in seen:
            seen.add(r)
            order.append(r)
    while len(order) < min(n, S):  # the rest uniformly over the sequence
        r = int(rng.integers(0, S))
        if r not in seen:
            seen.add(r)
            order.append(r)
    tap = order[:n_tap]
    return np.array(sorted(order), np.int64), np.array(sorted(tap), np.int64)


def golden_path(case: str) -> str:
    return os.path.join(HERE, f"{case}.npz")


def f32(a) -> np.ndarray:
    return np.asarray(a, np.float64).astype(np.float32)


def make(case: str) -> str:
    name, seed, gate_mean = CASES[case]
    t0 = time.time()
    wl = synth.make_workload(name, seed=seed, gate_mean=gate_mean)
    rows, tap_rows = sample_rows(wl.layout)
    x = wl.x.values()[0]
    ws = [oracle.weights_f64(b) for b in wl.blocks]
    del wl.blocks[:]
    out = {"rows": rows, "seq_len": np.int64(wl.layout.seq_len), "num_pad": np.int64(wl.layout.num_pad),
           "seed": np.int64(seed), "gate_mean": np.float64(gate_mean)}
    if len(ws) == 1:
        y, taps = ob.block_forward(x, wl.layout, ws[0], wl.dims, rows=rows, taps=True)
        sel = np.searchsorted(rows, tap_rows)
        out["tap_rows"] = tap_rows
        out["out"] = f32(y)
        out["x_mid"] = f32(taps["x_mid"])
        for k in ("attn_o", "attn_proj", "ffn_h", "ffn_out"):
            out[k] = f32(taps[k][sel])
    else:
        h = x
        for i, w in enumerate(ws[:-1]):
            h = ob.block_forward(h, wl.layout, w, wl.dims)
            if i == 0:
                out["block1_out"] = f32(h[rows])
            print(f"  {case}: block {i + 1} done ({time.time() - t0:.0f}s)", flush=True)
        out["out"] = f32(ob.block_forward(h, wl.layout, ws[-1], wl.dims, rows=rows))
    path = golden_path(case)
    np.savez_compressed(path, **out)
    print(f"{case}: wrote {path} ({os.path.getsize(path) / 2**20:.1f} MiB) in {time.time() - t0:.0f}s", flush=True)
    return path


if __name__ == "__main__":
    for c in (sys.argv[1:] or list(CASES)):
        make(c)
