"""GPU parity of the sign gradients (`blr_backward_signs`) with the f64 oracle.

G_U = diag(h) dy^T a diag(l) and G_V = diag(g) x^T db diag(l) (page:
`blr_backward` with sign state; tests `blr_sign_grad_matches_host`): relative
Frobenius error <= 3e-3 on every shape, the accumulate rule, the backward's
other outputs unchanged by the extra outputs, and the power-of-two staging
scale (invariance within the f16 range, failure without it).
"""
from __future__ import annotations

import numpy as np
import pytest

import binary_rank_linear_amd as blr
import oracle
import synth
from _gpu_util import TOL, check_shapes_fit, host, say, to_dev


def run_signs(d, gscale, dev, gu0=None, gv0=None, acc=False, keep_c=False):
    import torch
    t = to_dev(d, dev)
    y, ta, tc = blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], keep_c=keep_c)
    kw = {}
    if gu0 is not None:
        kw["grad_u"] = torch.from_numpy(np.ascontiguousarray(gu0, dtype=np.float32)).to(dev)
        kw["grad_v"] = torch.from_numpy(np.ascontiguousarray(gv0, dtype=np.float32)).to(dev)
    out = blr.blr_backward_signs(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], ta, tc, gscale,
                                 accumulate_signs=acc, **kw)
    torch.cuda.synchronize()
    return [host(v) for v in out]


SHAPES = [
    (128, 256, 256, 128),
    (70, 384, 256, 128),    # the page's test shape: 70 tokens
    (300, 512, 384, 256),   # ragged token tail (not a multiple of 32)
    (129, 256, 640, 384),
    (1000, 1024, 768, 512),
]


@pytest.mark.gpu
@pytest.mark.parametrize("M,d_in,d_out,r", SHAPES)
def test_sign_grads_match_oracle(dev, M, d_in, d_out, r):
    check_shapes_fit(M, d_in, d_out, r)
    d = synth.custom(M, d_in, d_out, r, seed=M + r, dy_sigma=1e-6)
    gs = float(d["gscale"])
    say(f"sign gradients M={M} d_in={d_in} d_out={d_out} r={r}")
    dh, dl, dg, dx, gu, gv = run_signs(d, gs, dev)
    GU, GV = oracle.sign_grads(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    assert oracle.rel_frobenius(gu, GU) < TOL
    assert oracle.rel_frobenius(gv, GV) < TOL
    # the rest of the backward is blr_backward's, bit for bit
    import torch
    t = to_dev(d, dev)
    _, ta, tc = blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"])
    b = blr.blr_backward(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], ta, tc, gs)
    torch.cuda.synchronize()
    for got, want in zip((dh, dl, dg, dx), b):
        assert np.array_equal(got, host(want))


@pytest.mark.gpu
def test_sign_grads_accumulate_and_c_tape(dev):
    M, d_in, d_out, r = 200, 256, 384, 128
    d = synth.custom(M, d_in, d_out, r, seed=5, dy_sigma=1e-6)
    gs = float(d["gscale"])
    rng = np.random.default_rng(9)
    GU, GV = oracle.sign_grads(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    gu0 = rng.standard_normal(GU.shape) * np.abs(GU).mean()
    gv0 = rng.standard_normal(GV.shape) * np.abs(GV).mean()
    say("sign gradients accumulate, with a c tape")
    _, _, _, _, gu, gv = run_signs(d, gs, dev, gu0=gu0, gv0=gv0, acc=True, keep_c=True)
    assert oracle.rel_frobenius(gu, gu0.astype(np.float32) + GU) < TOL
    assert oracle.rel_frobenius(gv, gv0.astype(np.float32) + GV) < TOL


@pytest.mark.gpu
def test_sign_grads_accumulate_over_token_ranges(dev):
    # d and r multiples of 256 and 35 steps of 32 tokens: the 256x256 tiles
    # with the tokens split in two ranges; the first writes (or adds to) the
    # output, the second's partial sums are added after it, in range order
    M, d_in, d_out, r = 1100, 512, 256, 256
    d = synth.custom(M, d_in, d_out, r, seed=23, dy_sigma=1e-6)
    gs = float(d["gscale"])
    rng = np.random.default_rng(4)
    GU, GV = oracle.sign_grads(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    gu0 = rng.standard_normal(GU.shape) * np.abs(GU).mean()
    gv0 = rng.standard_normal(GV.shape) * np.abs(GV).mean()
    say("sign gradients over two token ranges, accumulate and overwrite")
    _, _, _, _, gu, gv = run_signs(d, gs, dev, gu0=gu0, gv0=gv0, acc=True)
    assert oracle.rel_frobenius(gu, gu0.astype(np.float32) + GU) < TOL
    assert oracle.rel_frobenius(gv, gv0.astype(np.float32) + GV) < TOL
    _, _, _, _, gu, gv = run_signs(d, gs, dev, gu0=gu0, gv0=gv0, acc=False)
    assert oracle.rel_frobenius(gu, GU) < TOL
    assert oracle.rel_frobenius(gv, GV) < TOL


@pytest.mark.gpu
def test_sign_grads_gscale_invariance_and_negative_control(dev):
    M, d_in, d_out, r = 256, 512, 512, 256
    d = synth.custom(M, d_in, d_out, r, seed=11, dy_sigma=1e-7)
    GU, GV = oracle.sign_grads(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    say("sign gradients at two staging scales and at gscale 1")
    a = run_signs(d, 2.0 ** 22, dev)
    b = run_signs(d, 2.0 ** 20, dev)
    assert oracle.rel_frobenius(a[4], b[4]) < 1e-4 and oracle.rel_frobenius(a[5], b[5]) < 1e-4
    assert oracle.rel_frobenius(a[4], GU) < TOL and oracle.rel_frobenius(a[5], GV) < TOL
    c = run_signs(d, 1.0, dev)  # dy*h ~ 1e-7 falls into the f16 subnormals without the scale
    assert oracle.rel_frobenius(c[4], GU) > 10 * TOL


@pytest.mark.gpu
def test_sign_grads_attention_projection_full_size(dev):
    """The full attention-projection layer, where the tokens are split into
    four ranges whose partials are summed in range order: against the oracle,
    and bit-identical over two runs (the ranges finish in any order)."""
    w = synth.WORKLOADS[synth.HEADLINE]
    check_shapes_fit(w.M, w.d_in, w.d_out, w.r)
    d = synth.inputs(w)
    say(f"sign gradients at full size {w.name}")
    _, _, _, _, gu, gv = run_signs(d, w.gscale, dev)
    GU, GV = oracle.sign_grads(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    assert oracle.rel_frobenius(gu, GU) < TOL
    assert oracle.rel_frobenius(gv, GV) < TOL
    say(f"sign gradients at full size {w.name}: second run, bit for bit")
    _, _, _, _, gu2, gv2 = run_signs(d, w.gscale, dev)
    assert np.array_equal(gu, gu2) and np.array_equal(gv, gv2)


@pytest.mark.gpu
def test_sign_grads_reruns_are_bit_identical(dev):
    """Token ranges at a mid size (two of them), accumulate and overwrite:
    two runs give the same bits."""
    M, d_in, d_out, r = 1100, 512, 256, 256
    d = synth.custom(M, d_in, d_out, r, seed=31, dy_sigma=1e-6)
    gs = float(d["gscale"])
    g0 = np.random.default_rng(2).standard_normal((d_out, r)) * 1e-3
    v0 = np.random.default_rng(3).standard_normal((d_in, r)) * 1e-3
    for acc in (False, True):
        say(f"sign gradients rerun identity, accumulate={acc}")
        a = run_signs(d, gs, dev, gu0=g0, gv0=v0, acc=acc)
        b = run_signs(d, gs, dev, gu0=g0, gv0=v0, acc=acc)
        for k in range(6):
            assert np.array_equal(a[k], b[k]), k
