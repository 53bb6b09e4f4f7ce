"""Plain, slow, fp64 CPU oracle of the packed DiT block (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it. It shares no code with the HIP path and the HIP
path never imports it.
"""
from . import block, conditioning, edges, layout, step, w8a8  # noqa: F401
from .block import block_forward, chain_forward  # noqa: F401


def weights_f64(bw) -> dict:
    """Widen a synthetic block's stored weights to float64 (exact)."""
    import numpy as np
    return dict(w_qkv=bw.w_qkv.values(), w_out=bw.w_out.values(), w_gate_up=bw.w_gate_up.values(),
                w_down=bw.w_down.values(), q_norm=np.asarray(bw.q_norm, np.float64),
                k_norm=np.asarray(bw.k_norm, np.float64), adaln_table=np.asarray(bw.adaln_table, np.float64))
