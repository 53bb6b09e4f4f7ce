"""Write the expected values of the full-size parity tests.

    python tests/golden/make_golden.py [workload ...]

For each full-size workload (seed 0) this draws the synthetic inputs with
joint_video_audio_amd.synth, runs the fp64 oracle (oracle/) and stores, for
a fixed set of sampled packed rows, the block output (and, for single-block
workloads, the attention output of those rows; for the four-block chain,
also the first block's output). Values are stored as float16: their
rounding (<= 2^-11 relative) is far inside the float bar of the tests
(relative L2 1e-2, max-abs 5e-2). Nothing here touches the HIP path.
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

FULL = ["padless8k", "padded16k", "clip32k", "chain4x24k"]
N_SAMPLE = 32


def sample_rows(layout) -> np.ndarray:
    """Deterministic sample: ends, tile edges, each modality and padding rows."""
    S = layout.seq_len
    tags = layout.token_tags
    rows = {0, S - 1, 63, 64, 255, 256, S // 2}
    for want in (0, 1, 2, -1):
        idx = np.flatnonzero(tags == want)
        if idx.size:
            rows.update(int(i) for i in (idx[0], idx[-1], idx[idx.size // 2]))
    rng = np.random.default_rng(1234)
    while len(rows) < N_SAMPLE:
        rows.add(int(rng.integers(0, S)))
    return np.array(sorted(r for r in rows if 0 <= r < S)[:N_SAMPLE], np.int64)


def golden_path(name: str, seed: int = 0) -> str:
    return os.path.join(HERE, f"{name}_seed{seed}.npz")


def make(name: str, seed: int = 0) -> str:
    t0 = time.time()
    wl = synth.make_workload(name, seed=seed)
    rows = sample_rows(wl.layout)
    x = wl.x.values()[0]
    ws = [oracle.weights_f64(b) for b in wl.blocks]
    del wl.blocks[:]
    out = {"rows": rows, "seq_len": np.int64(wl.layout.seq_len), "num_pad": np.int64(wl.layout.num_pad)}
    if len(ws) == 1:
        y, taps = ob.block_forward(x, wl.layout, ws[0], wl.dims, rows=rows, taps=True)
        out["out"] = y.astype(np.float16)
        out["attn_o"] = taps["attn_o"].astype(np.float16)
    else:
        h = x
        for i, w in enumerate(ws[:-1]):
            h = ob.block_forward(h, wl.layout, w, wl.dims)
            if i == 0:
                out["block1_out"] = h[rows].astype(np.float16)
            print(f"  {name}: block {i + 1} done ({time.time() - t0:.0f}s)", flush=True)
        out["out"] = ob.block_forward(h, wl.layout, ws[-1], wl.dims, rows=rows).astype(np.float16)
    path = golden_path(name, seed)
    np.savez(path, **out)
    print(f"{name}: wrote {path} in {time.time() - t0:.0f}s", flush=True)
    return path


if __name__ == "__main__":
    for n in (sys.argv[1:] or FULL):
        make(n)
