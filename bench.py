"""Throughput of the packed DiT block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload clip32k]

A step is one forward pass of the whole block (all kernels: AdaLN, QKV
projection, q/k RMSNorm + RoPE, attention, output projection + gated
residual, AdaLN, SwiGLU FFN, down projection + gated residual) over one
packed sequence of synthetic inputs already resident in HBM. The default
workload is the clip-scale block: hidden 5376, 56 x 128 heads, FFN 14336,
32768 packed rows (1024 text, 1536 audio, 30208 video on a 16 x 32 x 59
grid), bf16. Prints one JSON line.

value = packed rows / s per block forward from the median of K steps, each
timed with a HIP event pair on the launch stream; TFLOP/s counts
algorithmic work only (GEMMs on non-padding rows, attention on same-document
pairs of non-padding rows). The output of the last timed step is compared,
in the same run, with the oracle's values at 256 sampled rows
(tests/golden/<workload>_seed<seed>.npz). A second pass of K steps records
an event pair around every launch (the library's MINIH3_PROFILE) for the
per-kernel times; the dominant kernel's roofline uses its average launch
time from that pass. A third, untimed pass samples the shader clock.
cpu_baseline times the fp64 oracle on a bounded sample of the workload.
table_build times, apart from the step, the build of one block's AdaLN
table from the workload's timestep values (time embeddings, then the bf16
AdaLN projection), with the projection's HBM roofline; edges times the
input projections into the packed sequence and the output heads (fp32);
w8a8 times the rotated W8A8 INT8 variant of the four projections beside the
bf16 ones (a separate variant: the headline step is bf16). other_workloads
times the other full-width workloads (8192 rows padless, 16384 rows with 640
padding rows, the four-block chain on 24576 + P rows) the same way, each with
its own same-run parity check; denoise_step times a clip-scale denoising step
(4 blocks) with and without unmerged adapters.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense)
HBM_PEAK_GBS = 8000.0


def flop_counts(dims, layout):
    """Algorithmic FLOP per block forward: (gemm, attention)."""
    import numpy as np
    D, W, F = dims.hidden, dims.num_heads * dims.head_dim, dims.ffn_dim
    real = int((np.asarray(layout.token_tags) != -1).sum())
    per_row = 2 * (D * 3 * W + W * D + D * 2 * F + F * D)
    gemm = per_row * real
    attn = 4 * dims.head_dim * dims.num_heads * real * real
    return gemm, attn


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attention_clip32k_traffic.md")
ATTENTION_SOURCE = os.path.join(ROOT, "joint_video_audio_amd", "csrc", "attention.hip")
TABLE_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "adaln_table_clip32k.md")
CONDITIONING_SOURCE = os.path.join(ROOT, "joint_video_audio_amd", "csrc", "conditioning.hip")


def measured_traffic(workload: str, summary: str = TRAFFIC_SUMMARY, source: str = ATTENTION_SOURCE):
    """HBM bytes per launch of a kernel from its committed FETCH_SIZE /
    WRITE_SIZE summary, or None when the summary covers another workload or
    another version of the kernel's source file."""
    import hashlib
    import re
    if workload != "clip32k" or not os.path.exists(summary):
        return None
    text = open(summary).read()
    m_sha = re.search(re.escape(os.path.basename(source)) + r" sha256: ([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch: ([0-9]+)", text)
    if not (m_sha and m_b):
        return None
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    return int(m_b.group(1)) if sha == m_sha.group(1) else None


def same_run_parity(workload: str, seed: int, out):
    """Compare the timed output at the oracle's sampled rows (written by
    tests/golden/make_golden.py from the fp64 oracle) with the bar of the
    parity tests: relative L2 <= 1e-2, max-abs <= 5e-2 beyond half a bf16
    ulp of the expected value. None when no expected values exist for the
    workload and seed."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", f"{workload}_seed{seed}.npz")
    if not os.path.exists(path):
        return None
    g = np.load(path, allow_pickle=False)
    rows = g["rows"]
    want = g["out"].astype(np.float64)
    got = out[0, torch_index(rows, out.device)].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 8)
    beyond = float((err - half_ulp).max())
    return {"expected": os.path.relpath(path, ROOT), "rows": int(rows.size), "rel_l2": rel,
            "max_abs": float(err.max()), "max_abs_beyond_half_bf16_ulp": beyond,
            "pass": bool(rel <= 1e-2 and beyond <= 5e-2 and np.all(np.isfinite(got)))}


def torch_index(a, device):
    import torch
    return torch.from_numpy(a).to(device)


def observed_clock(step, seconds: float = 3.0):
    """Mean shader clock over the XCDs while steps run back to back: a
    background thread reads `amd-smi metric -c` (GFX_i CLK lines) during
    about `seconds` of steps. None when amd-smi is not available."""
    import re
    import shutil
    import subprocess
    import threading
    import torch
    exe = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if not exe:
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                txt = subprocess.run([exe, "metric", "-c"], capture_output=True, text=True, timeout=10).stdout
            except Exception:  # pragma: no cover
                return
            clk, sec = [], None
            for line in txt.splitlines():
                h = re.match(r"\s*(GFX_\d+):", line)
                if h:
                    sec = h.group(1)
                    continue
                if re.match(r"\s*[A-Z]+_?\d*:\s*$", line):
                    sec = None
                c = re.match(r"\s*CLK:\s*([0-9.]+)\s*MHz", line)
                if c and sec:
                    clk.append(float(c.group(1)))
            if clk:
                samples.append(sum(clk) / len(clk))

    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds or (n < 200 and len(samples) < 2 and time.perf_counter() - t0 < 20):
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        n += 5
    stop.set()
    th.join(timeout=15)
    busy = [c for c in samples if c > 600.0]  # samples taken while the GPU ran (idle reads ~100 MHz)
    if not busy:
        return None
    return {"mean": round(sum(busy) / len(busy), 1), "min": round(min(busy), 1), "max": round(max(busy), 1),
            "samples": len(busy), "steps": n, "nominal": 2400.0,
            "source": "amd-smi metric -c, mean of the GFX_i clocks, sampled while the same step ran back to back "
                      "(a separate pass after the timed ones)"}


def cpu_baseline(wl, rows: int):
    """The oracle (fp64 numpy) timed on the first `rows` packed rows of the
    workload taken as their own sequence; scaled to rows/s of the full
    workload by FLOP per row."""
    import numpy as np
    import oracle
    from oracle import block as ob
    from joint_video_audio_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    L = wl.layout
    n = min(rows, L.seq_len)
    sub = synth.Layout(L.token_tags[:n], L.timestep_indices[:n], L.position_ids[:n],
                       L.video_indices[L.video_indices < n], L.audio_indices[L.audio_indices < n],
                       L.text_indices[L.text_indices < n])
    w = oracle.weights_f64(wl.blocks[0])
    x = wl.x.values()[0][:n]
    t0 = time.perf_counter()
    ob.block_forward(x, sub, w, wl.dims)
    t = time.perf_counter() - t0
    g_s, a_s = flop_counts(wl.dims, sub)
    g_f, a_f = flop_counts(wl.dims, L)
    flops_per_s = (g_s + a_s) / t
    rows_per_s = flops_per_s / ((g_f + a_f) / L.seq_len)
    return dict(value=rows_per_s, unit="rows/s", cores=int(cores), kind="oracle",
                sample=f"fp64 numpy oracle, full block on the first {n} packed rows of the workload as their own "
                       f"sequence ({t:.1f} s, {flops_per_s / 1e9:.1f} GFLOP/s); scaled to the full workload's rows/s "
                       f"by algorithmic FLOP per row")


def table_build(wl, seed: int, reps: int, warmup: int):
    """Time the AdaLN table build of one block for the workload's timestep
    values: the time embeddings (two-time on the clip workload, whose values
    are (sigma_now, sigma_next) pairs) and the bf16 AdaLN projection. HIP
    events bracket each call on the stream the library launches on."""
    import torch
    from joint_video_audio_amd import device as dv
    from joint_video_audio_amd import minih3 as m
    from joint_video_audio_amd import synth
    dims = wl.dims
    two = wl.name == "clip32k"
    cond = synth.make_conditioning(dims, two_time=two, seed=seed)
    cfg = dv.config_for(dims)
    tc = dv.time_config_for(cond)
    base = dv.time_mlp_for(cond.base)
    ep = dv.time_mlp_for(cond.endpoint) if two else None
    t = dv.f32(cond.t)
    r = dv.f32(cond.r) if two else None
    wp, bp = dv.to_device(cond.w_proj[0]), dv.to_device(cond.b_proj[0])
    n, E, D, T = dims.num_tvals, cond.embed_dim, dims.hidden, dims.num_tags
    emb = torch.empty(n, E, dtype=torch.float32, device="cuda")
    table = torch.empty(T, n, 6, D, dtype=torch.float32, device="cuda")
    ws_t = m.alloc_workspace(m.time_embed_workspace_bytes(tc, n))
    ws_a = m.alloc_workspace(m.adaln_table_workspace_bytes(cfg, E))

    def run():
        m.time_embed(tc, base, t, ep, r, cond.gate, out=emb, workspace=ws_t)
        m.adaln_table(cfg, emb, wp, bp, out=table, workspace=ws_a)

    for _ in range(warmup):
        run()
    st = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1, e2 in evs:
        e0.record(st)
        m.time_embed(tc, base, t, ep, r, cond.gate, out=emb, workspace=ws_t)
        e1.record(st)
        m.adaln_table(cfg, emb, wp, bp, out=table, workspace=ws_a)
        e2.record(st)
    torch.cuda.synchronize()
    te = sum(e0.elapsed_time(e1) for e0, e1, _ in evs) / reps
    ta = sum(e1.elapsed_time(e2) for _, e1, e2 in evs) / reps
    # algorithmic HBM bytes of the projection: bf16 weights and biases, fp32
    # time embeddings in, fp32 table out
    el = 2 if dims.dtype == "bf16" else 4
    nbytes = T * 6 * D * E * el + T * 6 * D * el + n * E * 4 + T * n * 6 * D * 4
    gbs = nbytes / (ta / 1e3) / 1e9
    return {"timestep_values": n, "two_time": two, "freq_dim": cond.freq_dim, "mlp_hidden": cond.hidden_dim,
            "embed_dim": E, "reps": reps, "time_embed_ms": round(te, 4), "adaln_table_ms": round(ta, 4),
            "roofline": {"kernel": "adaln_table", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(wl.name, TABLE_TRAFFIC_SUMMARY, CONDITIONING_SOURCE),
                         "algorithmic_bytes": nbytes, "avg_launch_ms": round(ta, 4)}}


FP32_MFMA_PEAK_TFLOPS = 157.3


def edges(wl, seed: int, reps: int, warmup: int):
    """Time the model edges on the workload's layout: the input projections
    with the scatter into the packed sequence (minih3_embed_inputs) and
    norm_out with the output heads on the gathered rows (minih3_output_heads).
    Both are fp32 contractions; HIP events bracket each call."""
    import torch
    from joint_video_audio_amd import device as dv
    from joint_video_audio_amd import minih3 as m
    from joint_video_audio_amd import synth
    L = wl.layout
    e = synth.make_edges(wl.dims, L, seed=seed)
    cfg = dv.config_for(wl.dims)
    lay = dv.layout_for(wl, batch=1)
    de = dv.edges_for(e)
    video, audio, text = dv.f32(e.video), dv.f32(e.audio), dv.to_device(e.text)
    x = torch.empty(1, L.seq_len, wl.dims.hidden, dtype=m.act_torch_dtype(cfg), device="cuda")
    ws = m.alloc_workspace(m.edges_workspace_bytes(cfg, de, L.seq_len))
    for _ in range(warmup):
        m.embed_inputs(cfg, lay, de, video, audio, text, x=x, workspace=ws)
        m.output_heads(cfg, lay, de, x, workspace=ws)
    st = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1, e2 in evs:
        e0.record(st)
        m.embed_inputs(cfg, lay, de, video, audio, text, x=x, workspace=ws)
        e1.record(st)
        m.output_heads(cfg, lay, de, x, workspace=ws)
        e2.record(st)
    torch.cuda.synchronize()
    t_in = sum(a.elapsed_time(b) for a, b, _ in evs) / reps
    t_out = sum(b.elapsed_time(c) for _, b, c in evs) / reps
    D, Cv, Ca = wl.dims.hidden, e.w_in.shape[1], e.w_ain.shape[1]
    nv, na = len(L.video_indices), len(L.audio_indices)
    flop = 2.0 * (nv * Cv + na * Ca) * D  # each direction
    tf_in, tf_out = flop / (t_in / 1e3) / 1e12, flop / (t_out / 1e3) / 1e12
    return {"video_rows": nv, "audio_rows": na, "video_channels": Cv, "audio_channels": Ca, "reps": reps,
            "embed_inputs_ms": round(t_in, 4), "output_heads_ms": round(t_out, 4),
            "roofline": {"kernel": "output_heads", "bound": "mfma", "achieved": round(tf_out, 1),
                         "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf_out / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                         "avg_launch_ms": round(t_out, 4)},
            "embed_inputs_tflops": round(tf_in, 1), "embed_inputs_frac": round(tf_in / FP32_MFMA_PEAK_TFLOPS, 4)}


INT8_MFMA_PEAK_TOPS = 5033.2  # 256 CU x 2.4 GHz x 8192 int8 ops/clk (dense)


def w8a8(reps: int, warmup: int, M: int = 32768):
    """Time the rotated W8A8 linear layer on the four projection shapes of the
    block at M packed rows (QKV, output, gate/up, down) beside the bf16
    projection on the same shapes, and the rotation + quantization of the
    activations. Synthetic N(0,1) activations and N(0,0.02) weights; HIP
    events bracket each call."""
    import torch
    from joint_video_audio_amd import minih3 as m
    shapes = {"qkv": (21504, 5376), "out": (5376, 7168), "gate_up": (28672, 5376), "down": (5376, 14336)}
    g = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    tot_i8 = tot_bf = tot_q = 0.0
    flop_all = 0.0
    for name, (N, K) in shapes.items():
        x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        qw, sw = m.rotate_quantize(w)
        qa, sa = m.rotate_quantize(x)
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

        def timed(fn):
            for _ in range(warmup):
                fn()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            for _ in range(reps):
                fn()
            e1.record(st)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        t_i8 = timed(lambda: m.linear_w8a8(qa, sa, qw, sw, out=out))
        t_bf = timed(lambda: m.linear(x, w, out=out))
        t_q = timed(lambda: m.rotate_quantize(x))
        flop = 2.0 * M * N * K
        res[name] = {"N": N, "K": K, "int8_ms": round(t_i8, 4), "bf16_ms": round(t_bf, 4),
                     "rotate_quantize_ms": round(t_q, 4), "int8_tops": round(flop / (t_i8 / 1e3) / 1e12, 1),
                     "bf16_tflops": round(flop / (t_bf / 1e3) / 1e12, 1)}
        tot_i8 += t_i8
        tot_bf += t_bf
        tot_q += t_q
        flop_all += flop
        del x, w, qw, qa, out
    tops = flop_all / (tot_i8 / 1e3) / 1e12
    res["rows"] = M
    res["total_int8_ms"] = round(tot_i8, 4)
    res["total_bf16_ms"] = round(tot_bf, 4)
    res["total_rotate_quantize_ms"] = round(tot_q, 4)
    res["roofline"] = {"kernel": "linear_w8a8", "bound": "mfma", "achieved": round(tops, 1),
                       "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOP/s", "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4),
                       "traffic": None, "avg_launch_ms": round(tot_i8 / 4, 4)}
    return res


def w8a8_block(wl, cfg, lay, blocks, x, steps: int, warmup: int):
    """The block forward with rotated W8A8 projections on the same workload
    and inputs as the headline step (a separate variant: the headline step is
    bf16). The weights are rotated and quantized once, outside the timing."""
    import torch
    from joint_video_audio_amd import minih3 as m
    qb = [m.DeviceBlockW8A8.from_block(b) for b in blocks]
    out = torch.empty_like(x)
    ws = m.alloc_workspace(m.workspace_bytes_w8a8(cfg, lay.batch, lay.seq_len))
    for _ in range(warmup):
        m.block_forward_w8a8(cfg, lay, qb, x, out=out, workspace=ws)
    torch.cuda.synchronize()
    m.profile_collect()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        m.block_forward_w8a8(cfg, lay, qb, x, out=out, workspace=ws, flags=m.PROFILE)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps / len(blocks)
    kern = {k: round(v[0] / max(v[1], 1), 4) for k, v in m.profile_collect().items() if v[1]}
    gemm, attn = flop_counts(wl.dims, wl.layout)
    return {"ms_per_block": round(ms, 4), "rows_per_s": round(lay.seq_len / (ms / 1e3), 1),
            "tflops_equivalent": round((gemm + attn) / (ms / 1e3) / 1e12, 1), "steps": steps,
            "kernel_avg_ms": kern,
            "note": "projection times include rotating and quantizing their input rows"}


def lora(reps: int, warmup: int, M: int = 32768, rank: int = 256):
    """Time the unmerged LoRA projection (rank 256) on the block's four
    projection shapes beside the plain projection: the low-rank part is
    rank / K more work plus building [x | s x A^T]."""
    import torch
    from joint_video_audio_amd import minih3 as m
    shapes = {"qkv": (21504, 5376), "out": (5376, 7168), "gate_up": (28672, 5376), "down": (5376, 14336)}
    g = torch.Generator(device="cuda").manual_seed(1)
    res = {}
    tot_l = tot_p = 0.0
    for name, (N, K) in shapes.items():
        a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        la = (torch.randn(rank, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        lb = (torch.randn(N, rank, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        packed = m.lora_pack_weight(w, lb)
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ws = m.alloc_workspace((M * rank + M * (K + rank)) * 2 + 1024)

        def timed(fn):
            for _ in range(warmup):
                fn()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            for _ in range(reps):
                fn()
            e1.record(st)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        t_l = timed(lambda: m.linear_lora(a, la, packed, 1.0, out=out, workspace=ws))
        t_p = timed(lambda: m.linear(a, w, out=out))
        res[name] = {"N": N, "K": K, "lora_ms": round(t_l, 4), "plain_ms": round(t_p, 4),
                     "overhead": round(t_l / t_p - 1.0, 4)}
        tot_l += t_l
        tot_p += t_p
        del a, w, la, lb, packed, out, ws
    res["rank"] = rank
    res["rows"] = M
    res["total_lora_ms"] = round(tot_l, 4)
    res["total_plain_ms"] = round(tot_p, 4)
    return res


def denoise_step(wl, reps: int, warmup: int, num_blocks: int = 4, rank: int = 256):
    """Time one denoising step at the workload's scale: input projections,
    `num_blocks` bf16 blocks each with an unmerged rank-256 adapter on its
    four projections, the output heads and the Euler update of the latents
    (minih3_denoise_step), beside the same step without adapters. Weights are
    drawn on the device (torch, seeded) with the distributions of the
    synthetic recipe; the layout, latents and edges are the workload's."""
    import numpy as np
    import torch
    from joint_video_audio_amd import device as dv
    from joint_video_audio_amd import minih3 as m
    from joint_video_audio_amd import synth
    dims = wl.dims
    cfg = dv.config_for(dims)
    lay = dv.layout_for(wl, batch=1)
    e = synth.make_edges(dims, wl.layout, seed=1)
    D, W, F = dims.hidden, dims.qkv_width, dims.ffn_dim
    g = torch.Generator(device="cuda").manual_seed(7)
    nrm = lambda *sh, std=0.02: (torch.randn(*sh, device="cuda", generator=g) * std).to(torch.bfloat16)  # noqa: E731
    blocks, loras = [], []
    for _ in range(num_blocks):
        tab = torch.randn(dims.num_tags, dims.num_tvals, 6, D, device="cuda", generator=g) * 0.1
        qn = 1 + 0.02 * torch.randn(128, device="cuda", generator=g)
        kn = 1 + 0.02 * torch.randn(128, device="cuda", generator=g)
        b = m.DeviceBlock(nrm(3 * W, D), nrm(D, W), nrm(2 * F, D), nrm(D, F), qn, kn, tab.contiguous())
        shapes = synth.lora_shapes(dims)
        a = {n: nrm(rank, K, std=K ** -0.5) for n, (N, K) in shapes.items()}
        bm = {n: nrm(N, rank) for n, (N, K) in shapes.items()}
        blocks.append(b)
        loras.append(m.DeviceBlockLora.from_block(b, a, bm))
    # the two-time workload's values are the (sigma_now, sigma_next) pairs of a k-point grid
    k = int(round(dims.num_tvals ** 0.5))
    assert k * k == dims.num_tvals, "a square number of timestep values (two-time pairs)"
    grid = (1.0 - np.arange(k) / k).astype(np.float32)
    v = np.arange(dims.num_tvals)
    now, nxt = dv.f32(grid[v // k]), dv.f32(grid[v % k])
    video0, audio0, text = dv.f32(e.video), dv.f32(e.audio), dv.to_device(e.text)
    de = dv.edges_for(e)
    res = {"blocks": num_blocks, "rank": rank, "rows": lay.seq_len, "reps": reps,
           "note": "weights drawn on the device (seeded torch) with the synthetic recipe's distributions"}
    for label, lo in (("with_adapters", loras), ("without_adapters", None)):
        video, audio = video0.clone(), audio0.clone()
        for _ in range(warmup):
            m.denoise_step(cfg, lay, blocks, de, now, nxt, video, audio, text, loras=lo, lora_scale=1.0)
        st = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        evs[0].record(st)
        for i in range(reps):
            m.denoise_step(cfg, lay, blocks, de, now, nxt, video, audio, text, loras=lo, lora_scale=1.0)
            evs[i + 1].record(st)
        torch.cuda.synchronize()
        ms = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]))
        res[label] = {"ms_per_step": round(ms, 3), "ms_per_block": round(ms / num_blocks, 3),
                      "rows_per_s_per_block": round(lay.seq_len / (ms / num_blocks / 1e3), 1)}
    res["adapter_overhead"] = round(res["with_adapters"]["ms_per_step"] / res["without_adapters"]["ms_per_step"] - 1,
                                    4)
    return res


def other_workloads(names, steps: int, warmup: int, seed: int = 0):
    """The other full-width workloads, each timed like the headline (median of
    `steps` per-step HIP event times, no per-kernel events) with its timed
    output compared with the oracle's sampled rows in the same run."""
    import numpy as np
    import torch
    from joint_video_audio_amd import device as dv
    from joint_video_audio_amd import minih3 as m
    from joint_video_audio_amd import synth
    res = {}
    for name in names:
        t0 = time.time()
        wl = synth.make_workload(name, seed=seed)
        cfg, lay, blocks, x = dv.upload(wl)
        out = torch.empty_like(x)
        ws = m.alloc_workspace(m.workspace_bytes(cfg, lay.batch, lay.seq_len))
        print(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        for _ in range(warmup):
            m.block_forward(cfg, lay, blocks, x, out=out, workspace=ws)
        st = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(st)
        for i in range(steps):
            m.block_forward(cfg, lay, blocks, x, out=out, workspace=ws)
            evs[i + 1].record(st)
        torch.cuda.synchronize()
        ms = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]))
        nb = len(blocks)
        gemm, attn = flop_counts(wl.dims, wl.layout)
        t_block = ms / 1e3 / nb
        tfl = (gemm + attn) / t_block / 1e12
        res[name] = {"seq_len": lay.seq_len, "pad_rows": wl.layout.num_pad, "blocks_per_step": nb,
                     "ms_per_step": round(ms, 4), "ms_per_block": round(ms / nb, 4),
                     "rows_per_s": round(lay.seq_len / t_block, 1), "tflops": round(tfl, 1),
                     "mfma_peak_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                     "parity": same_run_parity(name, seed, out)}
        del blocks, x, out, ws, wl
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="clip32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-table-build", action="store_true")
    ap.add_argument("--no-edges", action="store_true")
    ap.add_argument("--no-w8a8", action="store_true")
    ap.add_argument("--no-w8a8-block", action="store_true")
    ap.add_argument("--no-lora", action="store_true")
    ap.add_argument("--no-denoise-step", action="store_true")
    ap.add_argument("--no-clock", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="before the timed steps, copy a buffer of BYTES twice with torch (a plain copy kernel "
                         "of known size for scaling FETCH_SIZE / WRITE_SIZE counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the block is measured on a single "
              f"MI355X and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from joint_video_audio_amd import device as dv
    from joint_video_audio_amd import minih3 as m
    from joint_video_audio_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    m.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)

    if a.copy_calibration:
        src = torch.ones(a.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t0 = time.time()
    wl = synth.make_workload(a.workload, seed=a.seed)
    cfg, lay, blocks, x = dv.upload(wl)
    out = torch.empty_like(x)
    ws = m.alloc_workspace(m.workspace_bytes(cfg, lay.batch, lay.seq_len))
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s: {a.workload} S={lay.seq_len} "
          f"pads={wl.layout.num_pad} blocks={len(blocks)}", file=sys.stderr, flush=True)
    nb = len(blocks)

    for _ in range(a.warmup):
        m.block_forward(cfg, lay, blocks, x, out=out, workspace=ws)
    torch.cuda.synchronize()

    # headline: K steps, a HIP event pair around each on the launch stream
    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs[0].record(st)
    for i in range(a.steps):
        m.block_forward(cfg, lay, blocks, x, out=out, workspace=ws)
        evs[i + 1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps)]
    ms_step = float(np.median(step_ms))
    ms_mean = evs[0].elapsed_time(evs[-1]) / a.steps
    # the output of the last timed step against the oracle's sampled rows
    parity = same_run_parity(a.workload, a.seed, out)

    # per-kernel times: a second pass of K steps with the library's events
    # around every launch (MINIH3_PROFILE), on the same stream
    m.profile_collect()
    for _ in range(a.steps):
        m.block_forward(cfg, lay, blocks, x, out=out, workspace=ws, flags=m.PROFILE)
    torch.cuda.synchronize()
    kern = m.profile_collect()
    clock = None if a.no_clock else observed_clock(lambda: m.block_forward(cfg, lay, blocks, x, out=out,
                                                                           workspace=ws))

    gemm, attn = flop_counts(wl.dims, wl.layout)
    t_block = ms_step / 1e3 / nb
    rows_s = lay.seq_len / t_block
    tflops = (gemm + attn) / t_block / 1e12

    att_ms, att_n = kern["attention"]
    att_avg = att_ms / max(att_n, 1)
    att_tflops = attn / (att_avg / 1e3) / 1e12
    kernels = {k: round(v[0] / max(v[1], 1), 4) for k, v in kern.items() if v[1]}

    res = {
        "metric": "packed rows/s and TFLOP/s per block forward (hidden 5376, 56x128 heads) on 1 GPU",
        "value": round(rows_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dims.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) latents, N(0,0.02) weights, random-init AdaLN tables)",
        "config": {"workload": a.workload, "seq_len": lay.seq_len, "pad_rows": wl.layout.num_pad,
                   "blocks_per_step": nb, "hidden": wl.dims.hidden, "heads": wl.dims.num_heads,
                   "head_dim": wl.dims.head_dim, "ffn_dim": wl.dims.ffn_dim, "timestep_values": wl.dims.num_tvals,
                   "seed": a.seed},
        "ms_per_step_stat": "median of the per-step HIP event times",
        "ms_per_step_mean": round(ms_mean, 4),
        "ms_per_step_min": round(min(step_ms), 4),
        "ms_per_step_max": round(max(step_ms), 4),
        "tflops": round(tflops, 1),
        "mfma_peak_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "parity": parity,
        "clock_mhz": clock,
        "kernel_avg_ms": kernels,
        "kernel_avg_ms_pass": "a second pass of the same K steps with an event pair around every launch",
        "roofline": {"kernel": "attention", "bound": "mfma", "achieved": round(att_tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(a.workload),
                     "avg_launch_ms": round(att_avg, 4)},
    }
    if not a.no_table_build:
        res["table_build"] = table_build(wl, a.seed, reps=50, warmup=5)
    if not a.no_edges:
        res["edges"] = edges(wl, a.seed, reps=20, warmup=3)
    if not a.no_w8a8_block and wl.dims.dtype == "bf16":
        res["w8a8_block"] = w8a8_block(wl, cfg, lay, blocks, x, steps=10, warmup=2)
    if not a.no_w8a8 and a.workload == "clip32k":
        res["w8a8"] = w8a8(reps=10, warmup=2)
    if not a.no_lora and a.workload == "clip32k":
        res["lora"] = lora(reps=5, warmup=1)
    if not a.no_denoise_step and a.workload == "clip32k":
        del blocks, x, out, ws
        torch.cuda.empty_cache()
        res["denoise_step"] = denoise_step(wl, reps=3, warmup=1)
    if not a.no_other_workloads and a.workload == "clip32k":
        others = [n for n in ("padless8k", "padded16k", "chain4x24k")]
        res["other_workloads"] = other_workloads(others, steps=5, warmup=2, seed=a.seed)
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, a.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
