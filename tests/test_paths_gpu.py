"""GPU parity of the fused layer of several paths (`blr_forward_paths`,
`blr_backward_paths`; page: `blr_forward` / `blr_backward` over the paths of
a layer, y the sum of the paths) with the f64 oracle: relative Frobenius
error <= 3e-3 on y, the a tape, dx and every path's dh, dl, dg and sign
gradients, over ragged token counts and every fused-dh rank (128, 256, 512)
plus one that recomputes c per path (384); the accumulate rules; and one
path through the paths entry points equals the plain layer bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import binary_rank_linear_amd as blr
import oracle
import synth
from _gpu_util import TOL, check_shapes_fit, host, say, to_dev

SHAPES = [
    (300, 512, 384, 128, 2),   # ragged token tail
    (130, 256, 640, 256, 3),
    (513, 1024, 256, 512, 2),  # two rank tiles per path in the fused dh launch
    (200, 384, 256, 384, 2),   # dh from c recomputed per path (no fused launch at r = 384)
    (70, 256, 256, 128, 4),    # the most paths, the page's 70 tokens
    (300, 256, 512, 256, 2),   # F2 on the held activation, each path's h folded into its signs (256 ranks a path)
    (130, 512, 768, 128, 3),   # the same with 128 ranks a path, three paths
    (150, 512, 256, 384, 2),   # B2 on the held activation with 384 ranks a path
    (100, 256, 256, 256, 4),   # four paths of 256 ranks: a 1024-rank block in one workgroup
    (6100, 4096, 4096, 256, 2),  # F1 on 64 x 256 tiles of eight waves inside each path, the fused dh launch on
                                 # 256-rank tiles (one per path), a 20-row tail: every token against the oracle
]


def run_paths(d, gs, dev, signs=False, y0=None, dx0=None):
    import torch
    t = to_dev(d, dev)
    kw = {}
    if y0 is not None:
        kw = {"y": torch.from_numpy(np.ascontiguousarray(y0, dtype=np.float32)).to(dev), "accumulate_y": True}
    y, ta = blr.blr_forward_paths(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], **kw)
    kw = {}
    if dx0 is not None:
        kw = {"dx": torch.from_numpy(np.ascontiguousarray(dx0, dtype=np.float32)).to(dev), "accumulate_dx": True}
    dh, dl, dg, dx, gu, gv = blr.blr_backward_paths(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"],
                                                    ta, gs, signs=signs, **kw)
    torch.cuda.synchronize()
    out = {"y": host(y), "a": host(ta), "dh": host(dh), "dl": host(dl), "dg": host(dg), "dx": host(dx)}
    if signs:
        out["gu"], out["gv"] = host(gu), host(gv)
    return out


def want(d, y0=None, dx0=None, signs=False):
    y, a = oracle.forward_paths(d["x"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"], y0=y0,
                                accumulate=y0 is not None)
    dh, dl, dg, dx = oracle.backward_paths(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"],
                                           dx0=dx0, accumulate_dx=dx0 is not None)
    out = {"y": y, "a": a, "dh": dh, "dl": dl, "dg": dg, "dx": dx}
    if signs:
        out["gu"], out["gv"] = oracle.sign_grads_paths(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"],
                                                       d["g"])
    return out


def assert_close(got, ref, per_path=("dh", "dl", "dg", "gu", "gv")):
    errs = {}
    for k, v in got.items():
        if k in per_path:  # every path on its own
            for p in range(v.shape[0]):
                errs[f"{k}{p}"] = oracle.rel_frobenius(v[p], ref[k][p])
        else:
            errs[k] = oracle.rel_frobenius(v, ref[k])
    say("relative errors " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()))
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.gpu
@pytest.mark.parametrize("M,d_in,d_out,r,P", SHAPES)
def test_paths_match_oracle(dev, M, d_in, d_out, r, P):
    check_shapes_fit(M, d_in, d_out, P * r)
    d = synth.custom_paths(M, d_in, d_out, r, P, seed=8000 + M + P, dy_sigma=1e-6)
    gs = float(d["gscale"])
    say(f"paths parity M={M} d_in={d_in} d_out={d_out} r={r} P={P} gscale={gs}")
    assert_close(run_paths(d, gs, dev), want(d))


@pytest.mark.gpu
def test_paths_sign_grads(dev):
    M, d_in, d_out, r, P = 300, 512, 384, 256, 2
    d = synth.custom_paths(M, d_in, d_out, r, P, seed=8101, dy_sigma=1e-6)
    say(f"paths sign gradients M={M} r={r} P={P}")
    assert_close(run_paths(d, float(d["gscale"]), dev, signs=True), want(d, signs=True))


@pytest.mark.gpu
@pytest.mark.parametrize("M,d_in,d_out,r,P", [(200, 256, 384, 128, 3), (200, 256, 512, 256, 2),
                                               (130, 512, 256, 512, 2)])
def test_paths_accumulate_rules(dev, M, d_in, d_out, r, P):
    """y += sum_p h_p.c_p and dx += sum_p g_p.dx'_p when asked. Every shape
    takes the held-activation B2 over the paths in turn (d_in a multiple of
    256, P r <= 1024). The second takes the held-activation F2 with the
    paths' h folded in; the first (d_out = 384, not a multiple of 256) and the
    third (P r = 1024, past the held block) take the generic F2 with one
    flush per path."""
    d = synth.custom_paths(M, d_in, d_out, r, P, seed=8202 + r, dy_sigma=1e-6)
    R = np.random.default_rng(5)
    y0 = R.standard_normal((M, d_out)).astype(np.float32)
    dx0 = (R.standard_normal((M, d_in)) * 1e-5).astype(np.float32)
    say("paths accumulate rules")
    assert_close(run_paths(d, float(d["gscale"]), dev, y0=y0, dx0=dx0), want(d, y0=y0, dx0=dx0))


@pytest.mark.gpu
def test_paths_full_size_sampled(dev):
    """Two paths of 256 ranks at M=8192, d=4096, the launches the two-path
    benchmark line times (F2 in runs of four tiles on 8 waves with the paths'
    h folded in, B2 on the multi-path held-activation kernel in runs of eight
    tiles): with dy zero outside 48 sampled tokens, y, a and dx on the sample
    and every path's dh, dl, dg against the oracle run on the sample alone."""
    M, d_in, d_out, r, P = 8192, 4096, 4096, 256, 2
    check_shapes_fit(M, d_in, d_out, P * r)
    d = synth.custom_paths(M, d_in, d_out, r, P, seed=8505, dy_sigma=1e-6)
    R = np.random.default_rng(M)
    S = np.array(sorted(set(R.choice(M, size=45, replace=False).tolist()) | {0, M - 1, M - 65}))
    run = dict(d)
    run["dy"] = np.zeros_like(d["dy"])
    run["dy"][S] = d["dy"][S]
    say(f"paths full size M={M} d={d_in} r={r} P={P}, {len(S)} sampled tokens")
    got = run_paths(run, float(d["gscale"]), dev)
    got = {k: (v[S] if k in ("y", "a", "dx") else v) for k, v in got.items()}
    sub = {k: d[k] for k in ("bits_u", "bits_v", "h", "l", "g")}
    sub["x"], sub["dy"] = d["x"][S], d["dy"][S]
    assert_close(got, want(sub))


@pytest.mark.gpu
def test_one_path_equals_the_plain_layer(dev):
    """paths = 1 takes the plain layer's launches: bit-identical outputs."""
    import torch
    M, d_in, d_out, r = 300, 512, 384, 256
    d = synth.custom(M, d_in, d_out, r, seed=8303, dy_sigma=1e-6)
    gs = float(d["gscale"])
    t = to_dev(d, dev)
    say("one path through the paths entry points")
    y, ta, tc = blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"])
    b = blr.blr_backward(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], ta, tc, gs)
    p = {k: t[k][None] for k in ("bits_u", "bits_v", "h", "l", "g")}
    y1, ta1 = blr.blr_forward_paths(t["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    b1 = blr.blr_backward_paths(t["x"], t["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"], ta1, gs)
    torch.cuda.synchronize()
    assert np.array_equal(host(y1), host(y)) and np.array_equal(host(ta1), host(ta))
    for got, ref in zip(b1[:4], b):
        assert np.array_equal(host(got).reshape(-1), host(ref).reshape(-1))


@pytest.mark.gpu
def test_paths_reject_bad_arguments(dev):
    import torch
    d = synth.custom_paths(128, 256, 256, 128, 2, seed=8404)
    t = to_dev(d, dev)
    with pytest.raises(ValueError):  # path count of h and bits_u disagree
        blr.blr_forward_paths(t["x"], t["bits_u"][:1].contiguous(), t["bits_v"], t["h"], t["l"], t["g"])
    five = {k: torch.cat([t[k]] * 3)[:5].contiguous() for k in ("bits_u", "bits_v", "h", "l", "g")}
    with pytest.raises(blr.BlrError):  # more than four paths
        blr.blr_forward_paths(t["x"], five["bits_u"], five["bits_v"], five["h"], five["l"], five["g"],
                              ws=torch.empty(1 << 20, dtype=torch.uint8, device=dev))
