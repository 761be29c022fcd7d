"""GPU parity of the dense frozen linear (`blr_plane_linear`, page:
`plane_linear`) with the f64 oracle: relative Frobenius error <= 3e-3
over ragged token counts, the identity plane, and the staging scale."""
from __future__ import annotations

import numpy as np
import pytest

import binary_rank_linear_amd as blr
import oracle
from _gpu_util import TOL, host, say


def run(x, plane16, scale, dev):
    import torch
    y = blr.blr_plane_linear(torch.from_numpy(x).to(dev), torch.from_numpy(plane16.view(np.int16)).to(dev), scale)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.gpu
@pytest.mark.parametrize("M,n,k", [(1, 128, 128), (70, 256, 384), (300, 384, 256), (2048, 1024, 2048)])
def test_plane_linear_matches_oracle(dev, M, n, k):
    rng = np.random.default_rng(M + n)
    x = rng.standard_normal((M, k)).astype(np.float32)
    plane = (rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float16)
    say(f"plane_linear M={M} n={n} k={k}")
    got = run(x, plane, 1.0, dev)
    assert oracle.rel_frobenius(got, oracle.plane_linear(x, plane.view(np.uint16))) < TOL


@pytest.mark.gpu
def test_plane_linear_identity_and_scale(dev):
    k = 256
    rng = np.random.default_rng(3)
    x = rng.standard_normal((100, k)).astype(np.float32) * 1e-6
    eye = np.eye(k, dtype=np.float16)
    say("plane_linear identity, scale 2^20 and 1")
    y = run(x, eye, 2.0 ** 20, dev)
    assert oracle.rel_frobenius(y, x.astype(np.float64)) < 1e-3  # one f16 rounding of x * 2^20
    y1 = run(x, eye, 1.0, dev)  # 1e-6 lands in the f16 subnormals without the scale
    assert oracle.rel_frobenius(y1, x.astype(np.float64)) > 1e-3
