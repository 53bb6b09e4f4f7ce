"""The allocation-free AdaLN table build (GPU): minih3_adaln_table_noalloc
against the workspace entry point minih3_adaln_table, through the C ABI.

Two calls in a row on one device, the second with fewer timestep values
than the first, so that the second reads the library's shared scratch
after a larger call wrote it; each must equal the workspace entry point bit
for bit (the same kernels on the same inputs) and the fp64 oracle within the
bf16 bar. A request beyond the fixed scratch is refused before any work.
"""
import numpy as np
import pytest
import torch

from helpers import assert_close, gpu_available, to_np64
from joint_video_audio_amd import device as dv
from joint_video_audio_amd import minih3 as m
from joint_video_audio_amd import synth
from oracle import conditioning as oc

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def table_case(n, two_time, seed):
    dims = synth.ModelDims(num_tvals=n)
    c = synth.make_conditioning(dims, two_time=two_time, seed=seed)
    cfg = dv.config_for(dims)
    ep = c.endpoint.as_dict() if c.endpoint is not None else None
    emb_ref = oc.time_embedding(c.t, c.freq_dim, c.base.as_dict(), c.r, ep, c.gate)
    # the same fp32 embeddings feed both entry points
    emb = torch.from_numpy(emb_ref.astype(np.float32)).cuda()
    return dims, c, cfg, emb


def test_adaln_table_noalloc_equals_the_workspace_entry():
    print("adaln_table_noalloc: two calls, the second smaller", flush=True)
    for n, two, seed in ((64, True, 1), (5, False, 2)):
        dims, c, cfg, emb = table_case(n, two, seed)
        wp, bp = dv.to_device(c.w_proj[0]), dv.to_device(c.b_proj[0])
        got = torch.full((dims.num_tags, n, 6, dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
        m.adaln_table_noalloc(cfg, emb, wp, got, bp)
        ref = m.adaln_table(cfg, emb, wp, bp)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
        want = oc.adaln_table(emb.cpu().numpy().astype(np.float64), c.w_proj[0].values(), c.b_proj[0].values(),
                              dims.hidden)
        r, mx = assert_close(to_np64(got), want, f"adaln_table_noalloc n={n}")
        print(f"n={n}: equal to the workspace entry; vs oracle rel_l2={r:.3e} max_abs={mx:.3e}", flush=True)


def test_adaln_table_noalloc_refuses_beyond_its_scratch():
    # 200 timestep values x 2688 need 200 (padded to 256) x 2688 bf16 = 1.3 MiB > 1 MiB
    dims = synth.ModelDims(hidden=256, num_tvals=200)
    cfg = dv.config_for(dims)
    E = 2688
    emb = torch.zeros(200, E, dtype=torch.float32, device="cuda")
    wp = torch.zeros(dims.num_tags, 6 * dims.hidden, E, dtype=torch.bfloat16, device="cuda")
    out = torch.full((dims.num_tags, 200, 6, dims.hidden), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(m.Minih3Error) as e:
        m.adaln_table_noalloc(cfg, emb, wp, out)
    assert e.value.status == m.E_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was written
