"""GPU tests of the finite check (`blr_sumsq`, page: `sumsq`) and of the
power-of-two loss scale it drives (`all_finite`, `next_gscale`)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import binary_rank_linear_amd as blr
import oracle
import synth
from _gpu_util import TOL, host, say, to_dev


def f32_sumsq_bound(n: int, nparts: int = 64) -> float:
    """Relative error bound of the device sum: each thread adds about
    n / (nparts * 256) positive terms in f32, then an 8-level tree."""
    per_thread = max(1, -(-n // (nparts * 256)))
    return (per_thread + 8) * 2.0 ** -24 * 1.1


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, (1 << 20) + 3, 8192 * 4096])
def test_sumsq_matches_oracle(dev, n):
    import torch
    say(f"sumsq n={n}")
    a = np.random.default_rng(n % 1000).standard_normal(n).astype(np.float32)
    t = torch.from_numpy(a).to(dev)
    got = blr.blr_sumsq(t)
    want = oracle.sumsq(a)
    assert abs(got - want) <= f32_sumsq_bound(n) * want
    assert blr.blr_sumsq(t) == got  # deterministic


@pytest.mark.gpu
def test_sumsq_propagates_non_finite(dev):
    import torch
    say("sumsq with inf / nan")
    a = np.ones(100003, np.float32)
    for bad, check in ((np.inf, math.isinf), (np.nan, math.isnan), (3e20, math.isinf)):  # 3e20^2 overflows f32
        b = a.copy()
        b[77777] = bad
        assert check(blr.blr_sumsq(torch.from_numpy(b).to(dev)))
    assert blr.all_finite(torch.from_numpy(a).to(dev))


@pytest.mark.gpu
def test_dynamic_gscale_recovers_from_f16_overflow(dev):
    """Gradients of order 1 staged at 2^20 overflow f16 (max 65504): the
    finite check fails, the scale halves until the backward is finite, and
    that backward matches the oracle."""
    import torch
    M, d_in, d_out, r = 256, 512, 384, 128
    d = synth.custom(M, d_in, d_out, r, seed=13, dy_sigma=1.0)
    t = to_dev(d, dev)
    _, ta, tc = blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"])
    gs, tries = 2.0 ** 20, 0
    while True:
        say(f"backward at gscale 2^{int(math.log2(gs))}")
        dh, dl, dg, dx = blr.blr_backward(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], ta, tc,
                                          gs)
        ok = blr.all_finite(dh, dl, dg, dx)
        if ok:
            break
        gs = blr.next_gscale(gs, False)
        tries += 1
        assert tries < 30
    assert tries > 0  # the first scale did overflow
    want = oracle.backward(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    for got, w in zip((dh, dl, dg, dx), want):
        assert oracle.rel_frobenius(host(got), w) < TOL
