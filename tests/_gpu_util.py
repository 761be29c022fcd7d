"""Helpers shared by the GPU tests (not a test module)."""
from __future__ import annotations

import sys
import time

import numpy as np

TOL = 3e-3  # relative Frobenius bound on every float output (test `blr_layer_matches_host`)


def say(msg: str):
    """Name the case before each GPU step, flushed, so a failing run shows it."""
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(d: dict, dev):
    import torch
    out = {}
    for k, v in d.items():
        if isinstance(v, np.ndarray):
            if v.dtype == np.uint32:
                v = v.view(np.int32)
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    return out


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def check_shapes_fit(M, d_in, d_out, r):
    """Host-side check of the shape rule the kernels' grids assume."""
    assert M >= 1 and d_in % 128 == 0 and d_out % 128 == 0 and r % 128 == 0
