"""The allocation-free forward (`blr_forward_noalloc`) against blr_forward.

The same kernels run on the same inputs, so the outputs must agree bit for
bit: two calls in a row (the second smaller, so it reads only what it wrote
into the shared per-GPU scratch), with and without a c tape and with
accumulation, and a size whose transposed bitmap fills the scratch exactly.
The f64 oracle checks the first call as well (relative Frobenius error
<= 3e-3, the bar of the page's layer test).
"""
import numpy as np
import pytest

import binary_rank_linear_amd as blr
import oracle
import synth
from _gpu_util import TOL, check_shapes_fit, host, say, to_dev


def both(d, dev, acc=False, keep_c=False, y0=None):
    """blr_forward (with its workspace) and blr_forward_noalloc on the same
    inputs; returns the two (y, a, c) triples on the host."""
    import torch
    t = to_dev(d, dev)
    M, d_out = d["x"].shape[0], d["h"].shape[0]
    r = d["l"].shape[0]
    outs = []
    for noalloc in (False, True):
        y = torch.from_numpy(y0.copy()).to(dev) if y0 is not None else torch.empty((M, d_out), device=dev)
        ta = torch.empty((M, r), device=dev)
        tc = torch.empty((M, d_out), device=dev) if keep_c else None
        if noalloc:
            blr.blr_forward_noalloc(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], y, ta,
                                    accumulate_y=acc, tape_c=tc)
        else:
            blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], y=y, accumulate_y=acc,
                            tape_a=ta, tape_c=tc)
        torch.cuda.synchronize()
        outs.append((host(y), host(ta), None if tc is None else host(tc)))
    return outs


def assert_same(outs):
    (y0, a0, c0), (y1, a1, c1) = outs
    assert np.array_equal(y0, y1) and np.array_equal(a0, a1)
    assert (c0 is None) == (c1 is None)
    if c0 is not None:
        assert np.array_equal(c0, c1)


@pytest.mark.gpu
def test_noalloc_forward_matches_the_workspace_forward(dev):
    # two calls in a row on one GPU: the second with fewer tokens, a smaller
    # d_in and rank (a smaller transposed bitmap in the shared scratch)
    for (M, d_in, d_out, r) in [(8192, 4096, 4096, 512), (300, 512, 384, 256)]:
        check_shapes_fit(M, d_in, d_out, r)
        d = synth.custom(M, d_in, d_out, r, seed=77 + M, dy_sigma=1e-6)
        say(f"no-alloc forward M={M} d_in={d_in} d_out={d_out} r={r}")
        outs = both(d, dev)
        assert_same(outs)
        if M <= 300:
            y, a, _ = oracle.forward(d["x"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
            assert oracle.rel_frobenius(outs[1][0], y) <= TOL
            assert oracle.rel_frobenius(outs[1][1], a) <= TOL


@pytest.mark.gpu
def test_noalloc_forward_accumulate_and_c_tape(dev):
    M, d_in, d_out, r = 200, 256, 512, 256
    d = synth.custom(M, d_in, d_out, r, seed=5, dy_sigma=1e-6)
    y0 = np.random.default_rng(1).standard_normal((M, d_out)).astype(np.float32)
    say("no-alloc forward, accumulate y with a c tape")
    assert_same(both(d, dev, acc=True, keep_c=True, y0=y0))


@pytest.mark.gpu
def test_noalloc_forward_at_the_scratch_limit(dev):
    # r * d_in / 8 = 2048 * 16384 / 8: the whole scratch; then a smaller call
    M, d_in, d_out, r = 64, 16384, 256, 2048
    assert r * d_in // 8 == blr.NOALLOC_SCRATCH_BYTES
    d = synth.custom(M, d_in, d_out, r, seed=9, dy_sigma=1e-6)
    say(f"no-alloc forward at the scratch limit M={M} d_in={d_in} r={r}")
    assert_same(both(d, dev))
    d2 = synth.custom(130, 1024, 256, 128, seed=10, dy_sigma=1e-6)
    say("no-alloc forward after it, smaller")
    assert_same(both(d2, dev))


@pytest.mark.gpu
def test_noalloc_forward_rejects_past_the_scratch(dev):
    import torch
    M, d_in, d_out, r = 64, 16384 + 128, 256, 2048
    f = dict(device=dev)
    x = torch.zeros((M, d_in), **f)
    bu = torch.zeros((d_out, r // 32), dtype=torch.int32, **f)
    bv = torch.zeros((d_in, r // 32), dtype=torch.int32, **f)
    h, l, g = torch.zeros(d_out, **f), torch.zeros(r, **f), torch.zeros(d_in, **f)
    y, ta = torch.full((M, d_out), 7.0, **f), torch.full((M, r), 7.0, **f)
    say("no-alloc forward past the scratch: rejected, outputs untouched")
    with pytest.raises(blr.BlrError) as e:
        blr.blr_forward_noalloc(x, bu, bv, h, l, g, y, ta)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((ta == 7.0).all())
