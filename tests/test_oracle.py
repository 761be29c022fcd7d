"""Pins of the f64 oracle against facts outside it (CPU only).

Each check is chosen so that a plausible slip in the oracle (a dropped
factor, a wrong sign, a transposed operand, a wrong bit index or word
stride, a missing accumulate) fails at least one of them:

* bit convention: numpy's own `unpackbits` (little bit order) on the words,
  unit bitmaps, word-edge ranks, ragged last word;
* forward: the dense layer matrix W^ = diag(h) S_U diag(l) S_V^T diag(g)
  materialised with numpy matmul, rank-one closed forms, a hand-worked
  example, the accumulate rule;
* backward: exact central differences (y is linear in each of x, h, l, g
  separately, so the difference quotient has no truncation term), the dense
  form dx = dy W^, Euler identities sum(theta * dL/dtheta) = L;
* the sign-flip identity of test `blr_sign_flip_exact` on the page.

Source: cortiq-engine "src/gpu_wgpu/train_mm.rs" (0.8.21): module doc block,
`expand` shader, `blr_forward`, `blr_backward`, tests
`blr_layer_matches_host` and `blr_sign_flip_exact`.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unpack_signs(bits: np.ndarray, rows: int, r: int) -> np.ndarray:
    """+-1 signs from numpy's bit unpacking (independent of the oracle)."""
    b = np.ascontiguousarray(bits, dtype="<u4").reshape(rows, -1).view(np.uint8)
    u = np.unpackbits(b, axis=1, bitorder="little")[:, :r]
    return np.where(u == 1, 1.0, -1.0)


def dense_w(p) -> np.ndarray:
    d_out, d_in, r = p["h"].size, p["g"].size, p["l"].size
    SU = unpack_signs(p["bits_u"], d_out, r)
    SV = unpack_signs(p["bits_v"], d_in, r)
    h, l, g = (p[k].astype(np.float64) for k in ("h", "l", "g"))
    return (h[:, None] * SU) @ (l[:, None] * SV.T) * g[None, :]


def small(M, d_in, d_out, r, seed, dy_sigma=1.0):
    d = synth.custom(M, d_in, d_out, r, seed, dy_sigma=dy_sigma, l_hi=1.0)
    return d


# ---------------------------------------------------------------- decode --

@pytest.mark.parametrize("rows,r", [(3, 32), (5, 40), (4, 128), (2, 1), (7, 97)])
def test_decode_matches_numpy_unpackbits(rows, r):
    bits = synth.sign_bits(rows, r, 7 + r)
    S = oracle.decode_signs(bits, rows, r)
    assert np.array_equal(S, unpack_signs(bits, rows, r))


def test_decode_unit_bitmaps():
    rows, r = 6, 128
    W = r // 32
    assert np.all(oracle.decode_signs(np.zeros((rows, W), np.uint32), rows, r) == -1.0)
    assert np.all(oracle.decode_signs(np.full((rows, W), 0xFFFFFFFF, np.uint32), rows, r) == 1.0)
    bits = np.zeros((rows, W), np.uint32)
    bits[4, 1] = 1 << 5  # row 4, word 1, bit 5 -> rank 37
    S = oracle.decode_signs(bits, rows, r)
    want = -np.ones((rows, r))
    want[4, 37] = 1.0
    assert np.array_equal(S, want)


@pytest.mark.parametrize("k", [0, 31, 32, 63, 64, 95, 96, 127])
def test_decode_word_edges(k):
    rows, r = 3, 128
    bits = np.zeros((rows, r // 32), np.uint32)
    bits[2, k // 32] |= np.uint32(1 << (k % 32))
    S = oracle.decode_signs(bits, rows, r)
    assert S[2, k] == 1.0 and np.sum(S == 1.0) == 1


def test_decode_ignores_bits_past_rank():
    rows, r = 2, 40  # two words per row, the last one holds ranks 32..39
    bits = np.zeros((rows, 2), np.uint32)
    bits[:, 1] = 0xFFFFFF00  # only bits >= 8 of word 1: ranks >= 40, outside r
    assert np.all(oracle.decode_signs(bits, rows, r) == -1.0)
    bits[:, 1] = 0xFFFFFFFF
    S = oracle.decode_signs(bits, rows, r)
    assert np.all(S[:, 32:] == 1.0) and np.all(S[:, :32] == -1.0)


def test_pack_then_decode_roundtrip():
    """The page packs a sign s > 0 as bit (j % 32) of word j / 32 (its `pack`
    closure); numpy packbits with little bit order writes the same words."""
    rng = np.random.default_rng(3)
    rows, r = 9, 96
    s = np.where(rng.random((rows, r)) < 0.5, 1.0, -1.0)
    words = np.packbits((s > 0).astype(np.uint8), axis=1, bitorder="little").view("<u4")
    assert np.array_equal(oracle.decode_signs(words.astype(np.uint32), rows, r), s)


@pytest.mark.parametrize("rows,r", [(4, 32), (6, 40), (128, 128)])
def test_expand_planes_patterns(rows, r):
    bits = synth.sign_bits(rows, r, 11)
    pl, plt = oracle.expand_planes(bits, rows, r)
    assert set(np.unique(pl)) <= {0x3C00, 0xBC00}
    assert np.array_equal(pl.view(np.float16).astype(np.float64), unpack_signs(bits, rows, r))
    assert np.array_equal(plt, pl.T)


# --------------------------------------------------------------- forward --

def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_2x2.json")) as f:
        e = json.load(f)
    bu = np.array(e["bits_u"], np.uint32).reshape(2, 1)
    bv = np.array(e["bits_v"], np.uint32).reshape(2, 1)
    x, dy = np.array(e["x"]), np.array(e["dy"])
    h, l, g = np.array(e["h"]), np.array(e["l"]), np.array(e["g"])
    y, a, c = oracle.forward(x, bu, bv, h, l, g)
    assert np.array_equal(a, e["a"]) and np.array_equal(c, e["c"]) and np.array_equal(y, e["y"])
    dh, dl, dg, dx = oracle.backward(x, dy, bu, bv, h, l, g)
    for got, key in [(dh, "dh"), (dl, "dl"), (dg, "dg"), (dx, "dx")]:
        assert np.array_equal(got, np.array(e[key])), key


@pytest.mark.parametrize("M,d_in,d_out,r", [(5, 7, 6, 40), (1, 3, 2, 1), (70, 33, 65, 64), (130, 16, 24, 33)])
def test_forward_matches_dense(M, d_in, d_out, r):
    p = small(M, d_in, d_out, r, 100 + M)
    y, a, c = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    want = p["x"].astype(np.float64) @ dense_w(p).T
    assert oracle.rel_frobenius(y, want) < 1e-12
    # the tape is h-free: y = h * c exactly in f64 up to one rounding
    assert np.allclose(y, p["h"].astype(np.float64)[None, :] * c, rtol=1e-15, atol=0)


def test_forward_rank_one_closed_forms():
    M, d_in, d_out, r = 4, 10, 12, 64
    p = small(M, d_in, d_out, r, 5)
    ones_u = np.full((d_out, 2), 0xFFFFFFFF, np.uint32)
    ones_v = np.full((d_in, 2), 0xFFFFFFFF, np.uint32)
    zero_u, zero_v = np.zeros_like(ones_u), np.zeros_like(ones_v)
    x, h, l, g = (p[k].astype(np.float64) for k in ("x", "h", "l", "g"))
    xg = x @ g  # sum_j g_j x[t][j]
    base = h[None, :] * l.sum() * xg[:, None]
    for bu, bv, sign in [(ones_u, ones_v, 1), (zero_u, zero_v, 1), (ones_u, zero_v, -1), (zero_u, ones_v, -1)]:
        y, a, _ = oracle.forward(p["x"], bu, bv, p["h"], p["l"], p["g"])
        assert np.allclose(y, sign * base, rtol=1e-12, atol=1e-12)
        # a[t][k] is +-sum_j x g for every rank k
        sa = 1 if bv is ones_v else -1
        assert np.allclose(a, sa * np.repeat(xg[:, None], r, axis=1), rtol=1e-12, atol=1e-12)


def test_forward_single_sign_column():
    """All S_V signs -1 except row j0 (+1 on every rank): a[t][k] =
    -sum_j x g + 2 x[t][j0] g[j0] for every k."""
    M, d_in, d_out, r = 3, 9, 5, 32
    p = small(M, d_in, d_out, r, 8)
    bv = np.zeros((d_in, 1), np.uint32)
    bv[6, 0] = 0xFFFFFFFF
    _, a, _ = oracle.forward(p["x"], p["bits_u"], bv, p["h"], p["l"], p["g"])
    x, g = p["x"].astype(np.float64), p["g"].astype(np.float64)
    want = -(x @ g) + 2 * x[:, 6] * g[6]
    assert np.allclose(a, np.repeat(want[:, None], r, axis=1), rtol=1e-12, atol=1e-12)


def test_forward_accumulate_rule():
    """`blr_forward` overwrites y for path 0 and adds for later paths."""
    p = small(6, 20, 18, 32, 9)
    y0 = np.random.default_rng(1).standard_normal((6, 18))
    y_over, _, _ = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"], y0=y0, accumulate=False)
    y_acc, _, _ = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"], y0=y0, accumulate=True)
    y_new, _, _ = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    assert np.array_equal(y_over, y_new)
    assert np.allclose(y_acc, y0 + y_new, rtol=1e-14, atol=1e-14)


# -------------------------------------------------------------- backward --

def loss(p, x=None, h=None, l=None, g=None):
    x = p["x"] if x is None else x
    h = p["h"] if h is None else h
    l = p["l"] if l is None else l
    g = p["g"] if g is None else g
    y, _, _ = oracle.forward(x, p["bits_u"], p["bits_v"], h, l, g, tape=False)
    return float(np.sum(p["dy"].astype(np.float64) * y))


def central(p, name, eps=0.25):
    base = p[name].astype(np.float64)
    out = np.empty(base.size)
    for e in range(base.size):
        plus, minus = base.copy().reshape(-1), base.copy().reshape(-1)
        plus[e] += eps
        minus[e] -= eps
        lp = loss(p, **{name: plus.reshape(base.shape)})
        lm = loss(p, **{name: minus.reshape(base.shape)})
        out[e] = (lp - lm) / (2 * eps)
    return out.reshape(base.shape)


@pytest.mark.parametrize("M,d_in,d_out,r", [(3, 5, 4, 33), (2, 8, 6, 64)])
def test_backward_central_differences(M, d_in, d_out, r):
    p = small(M, d_in, d_out, r, 20 + r)
    dh, dl, dg, dx = oracle.backward(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    for got, name in [(dh, "h"), (dl, "l"), (dg, "g"), (dx, "x")]:
        fd = central(p, name)
        assert oracle.rel_frobenius(got, fd) < 1e-10, name


@pytest.mark.parametrize("M,d_in,d_out,r", [(70, 33, 65, 64), (129, 40, 24, 96), (1, 1, 1, 1)])
def test_backward_dense_and_euler(M, d_in, d_out, r):
    p = small(M, d_in, d_out, r, 300 + M)
    x, dy = p["x"].astype(np.float64), p["dy"].astype(np.float64)
    Wd = dense_w(p)
    dh, dl, dg, dx = oracle.backward(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    assert oracle.rel_frobenius(dx, dy @ Wd) < 1e-12
    L = float(np.sum(dy * (x @ Wd.T)))
    for got, theta in [(dh, p["h"]), (dl, p["l"]), (dg, p["g"]), (dx, p["x"])]:
        s = float(np.sum(got * theta.astype(np.float64)))
        assert abs(s - L) <= 1e-10 * max(1.0, abs(L))


def test_backward_accumulate_rules():
    """dh, dl, dg always accumulate; dx is overwritten unless asked to add."""
    p = small(67, 12, 10, 32, 41)
    args = (p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    dh, dl, dg, dx = oracle.backward(*args)
    R = np.random.default_rng(2)
    dh0, dl0, dg0, dx0 = R.standard_normal(10), R.standard_normal(32), R.standard_normal(12), R.standard_normal((67, 12))
    dh2, dl2, dg2, dx2 = oracle.backward(*args, dh0=dh0, dl0=dl0, dg0=dg0, dx0=dx0)
    assert np.allclose(dh2, dh0 + dh, rtol=1e-13, atol=1e-13)
    assert np.allclose(dl2, dl0 + dl, rtol=1e-13, atol=1e-13)
    assert np.allclose(dg2, dg0 + dg, rtol=1e-13, atol=1e-13)
    assert np.array_equal(dx2, dx)
    _, _, _, dx3 = oracle.backward(*args, dx0=dx0, accumulate_dx=True)
    assert np.allclose(dx3, dx0 + dx, rtol=1e-13, atol=1e-13)


def test_backward_is_deterministic_and_tokenwise():
    """Rerunning gives identical bits; the token sums are over exactly the
    tokens given (splitting the tokens and adding the halves agrees)."""
    p = small(150, 20, 16, 32, 77)
    args = (p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    r1 = oracle.backward(p["x"], p["dy"], *args)
    r2 = oracle.backward(p["x"], p["dy"], *args)
    for u, v in zip(r1, r2):
        assert np.array_equal(u, v)
    a = oracle.backward(p["x"][:70], p["dy"][:70], *args)
    b = oracle.backward(p["x"][70:], p["dy"][70:], *args)
    for i in range(3):
        assert np.allclose(r1[i], a[i] + b[i], rtol=1e-12, atol=1e-15)
    assert np.array_equal(r1[3], np.concatenate([a[3], b[3]]))


# ------------------------------------------------------- sign-flip identity --

def test_sign_flip_identity():
    """With L = 1/2 ||y - y*||^2, flipping S_U[i][k] changes L by exactly
    -2 s G_U[i][k] + 2 h_i^2 l_k^2 sum_t a_tk^2, and S_V[j][k] by
    -2 s G_V[j][k] + 2 g_j^2 l_k^2 (sum_t x_tj^2)(sum_i h_i^2), where
    G_U = diag(h) dy^T a diag(l), G_V = diag(g) x^T b diag(l), dy = y - y*,
    b = (dy*h) S_U (test `blr_sign_flip_exact`). Each flip rewrites one bit
    and reruns the oracle forward, so this pins the bit -> (row, rank) map."""
    M, d_in, d_out, r = 20, 48, 40, 128
    p = synth.exact_grid(M, d_in, d_out, r, 31)
    x, h, l, g = (p[k].astype(np.float64) for k in ("x", "h", "l", "g"))
    y0, a, _ = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    ystar = y0 + 0.7 * np.sqrt(np.mean(y0 ** 2)) * np.random.default_rng(71).standard_normal(y0.shape)
    dy = y0 - ystar
    SU = unpack_signs(p["bits_u"], d_out, r)
    SV = unpack_signs(p["bits_v"], d_in, r)
    b = (dy * h[None, :]) @ SU
    GU = h[:, None] * (dy.T @ a) * l[None, :]
    GV = g[:, None] * (x.T @ b) * l[None, :]
    L0 = 0.5 * np.sum((y0 - ystar) ** 2)
    picks = [(0, 0), (1, 31), (2, 32), (39, 127), (17, 63), (30, 64), (20, 95), (5, 96)]
    worst = 0.0
    for side in ("U", "V"):
        for (i, k) in picks:
            bu, bv = p["bits_u"].copy(), p["bits_v"].copy()
            if side == "U":
                s0 = SU[i, k]
                bu[i, k // 32] ^= np.uint32(1 << (k % 32))
                pred = -2 * s0 * GU[i, k] + 2 * h[i] ** 2 * l[k] ** 2 * np.sum(a[:, k] ** 2)
                scale = 2 * abs(GU[i, k]) + 2 * h[i] ** 2 * l[k] ** 2 * np.sum(a[:, k] ** 2)
            else:
                s0 = SV[i, k]
                bv[i, k // 32] ^= np.uint32(1 << (k % 32))
                quad = 2 * g[i] ** 2 * l[k] ** 2 * np.sum(x[:, i] ** 2) * np.sum(h ** 2)
                pred = -2 * s0 * GV[i, k] + quad
                scale = 2 * abs(GV[i, k]) + quad
            y1, _, _ = oracle.forward(p["x"], bu, bv, p["h"], p["l"], p["g"], tape=False)
            dL = 0.5 * np.sum((y1 - ystar) ** 2) - L0
            worst = max(worst, abs(dL - pred) / scale)
    assert worst < 1e-9


def test_sign_flip_identity_catches_wrong_word_stride():
    """Negative control: flipping the bit one word over (a plausible stride
    slip) breaks the identity by O(1)."""
    M, d_in, d_out, r = 12, 24, 20, 128
    p = synth.exact_grid(M, d_in, d_out, r, 32)
    h, l = p["h"].astype(np.float64), p["l"].astype(np.float64)
    y0, a, _ = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    ystar = y0 + np.random.default_rng(5).standard_normal(y0.shape) * np.std(y0)
    dy = y0 - ystar
    SU = unpack_signs(p["bits_u"], d_out, r)
    GU = h[:, None] * (dy.T @ a) * l[None, :]
    i, k = 3, 40
    bu = p["bits_u"].copy()
    bu[i, k // 32 + 1] ^= np.uint32(1 << (k % 32))  # wrong word
    y1, _, _ = oracle.forward(p["x"], bu, p["bits_v"], p["h"], p["l"], p["g"], tape=False)
    dL = 0.5 * np.sum((y1 - ystar) ** 2) - 0.5 * np.sum(dy ** 2)
    quad = 2 * h[i] ** 2 * l[k] ** 2 * np.sum(a[:, k] ** 2)
    pred = -2 * SU[i, k] * GU[i, k] + quad
    assert abs(dL - pred) / (2 * abs(GU[i, k]) + quad) > 1e-3


# ----------------------------------------------------------- input module --

def test_workloads_shapes_and_scales():
    for w in synth.WORKLOADS.values():
        assert w.d_in % 128 == 0 and w.d_out % 128 == 0 and w.r % 128 == 0
        assert w.gscale > 0 and np.log2(w.gscale) == int(np.log2(w.gscale))
    w = synth.WORKLOADS[synth.HEADLINE]
    assert (w.M, w.d_in, w.d_out, w.r) == (8192, 4096, 4096, 512)
    assert w.gscale == 2.0 ** 19
    assert synth.WORKLOADS["mlp_up_8192x4096x12288_r1024"].gscale == 2.0 ** 22
    t = synth.inputs(synth.WORKLOADS[synth.SMALL])
    assert t["x"].dtype == np.float32 and t["bits_u"].shape == (256, 4) and t["bits_u"].dtype == np.uint32
    assert np.all((t["h"] >= 0.5) & (t["h"] <= 1.5)) and np.all((t["l"] >= 0) & (t["l"] <= 0.1))
    # same seed, same numbers
    assert np.array_equal(t["x"], synth.inputs(synth.WORKLOADS[synth.SMALL])["x"])


# ------------------------------------------------------- sign gradients --

def _relaxed_loss(p, dy, SU, SV):
    """sum(dy * y) with the sign matrices taken as real matrices (dense)."""
    x, h, l, g = (p[k].astype(np.float64) for k in ("x", "h", "l", "g"))
    W = (h[:, None] * SU) @ (l[:, None] * SV.T) * g[None, :]
    return float(np.sum(dy * (x @ W.T)))


def test_sign_grads_match_relaxed_central_differences():
    """G_U and G_V are the gradients of L = sum(dy * y) with respect to the
    entries of S_U and S_V taken as real numbers; L is linear in each entry,
    so the central difference quotient of the dense form is exact."""
    M, d_in, d_out, r = 6, 10, 9, 40
    p = small(M, d_in, d_out, r, seed=81)
    dy = p["dy"].astype(np.float64)
    SU = unpack_signs(p["bits_u"], d_out, r)
    SV = unpack_signs(p["bits_v"], d_in, r)
    GU, GV = oracle.sign_grads(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    eps = 0.25
    fd_u = np.empty_like(GU)
    for i in range(d_out):
        for k in range(r):
            E = np.zeros_like(SU)
            E[i, k] = eps
            fd_u[i, k] = (_relaxed_loss(p, dy, SU + E, SV) - _relaxed_loss(p, dy, SU - E, SV)) / (2 * eps)
    fd_v = np.empty_like(GV)
    for j in range(d_in):
        for k in range(r):
            E = np.zeros_like(SV)
            E[j, k] = eps
            fd_v[j, k] = (_relaxed_loss(p, dy, SU, SV + E) - _relaxed_loss(p, dy, SU, SV - E)) / (2 * eps)
    assert oracle.rel_frobenius(GU, fd_u) < 1e-12
    assert oracle.rel_frobenius(GV, fd_v) < 1e-12


def test_sign_grads_flip_identity():
    """The page's flip identity with the oracle's G_U, G_V: flipping one bit
    and rerunning the oracle forward changes L = 1/2 ||y - y*||^2 by exactly
    -2 s G + (the quadratic term), at word-edge ranks."""
    M, d_in, d_out, r = 16, 40, 36, 128
    p = synth.exact_grid(M, d_in, d_out, r, 33)
    x, h, l, g = (p[k].astype(np.float64) for k in ("x", "h", "l", "g"))
    y0, a, _ = oracle.forward(p["x"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    ystar = y0 + 0.5 * np.sqrt(np.mean(y0 ** 2)) * np.random.default_rng(83).standard_normal(y0.shape)
    dy = y0 - ystar
    GU, GV = oracle.sign_grads(p["x"], dy, p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    SU = unpack_signs(p["bits_u"], d_out, r)
    SV = unpack_signs(p["bits_v"], d_in, r)
    L0 = 0.5 * np.sum(dy ** 2)
    worst = 0.0
    for side in ("U", "V"):
        for (i, k) in [(0, 0), (3, 31), (7, 32), (35, 127), (11, 63), (20, 64), (2, 95), (9, 96)]:
            bu, bv = p["bits_u"].copy(), p["bits_v"].copy()
            if side == "U":
                bu[i, k // 32] ^= np.uint32(1 << (k % 32))
                quad = 2 * h[i] ** 2 * l[k] ** 2 * np.sum(a[:, k] ** 2)
                pred, scale = -2 * SU[i, k] * GU[i, k] + quad, 2 * abs(GU[i, k]) + quad
            else:
                bv[i, k // 32] ^= np.uint32(1 << (k % 32))
                quad = 2 * g[i] ** 2 * l[k] ** 2 * np.sum(x[:, i] ** 2) * np.sum(h ** 2)
                pred, scale = -2 * SV[i, k] * GV[i, k] + quad, 2 * abs(GV[i, k]) + quad
            y1, _, _ = oracle.forward(p["x"], bu, bv, p["h"], p["l"], p["g"], tape=False)
            worst = max(worst, abs(0.5 * np.sum((y1 - ystar) ** 2) - L0 - pred) / scale)
    assert worst < 1e-9


def test_sign_grads_euler_identities_against_the_backward():
    """sum_k S_U[i][k] G_U[i][k] = h_i dh_i and sum_k S_V[j][k] G_V[j][k] =
    g_j dg_j (y is linear in S_U and in S_V, so scaling a row of S scales the
    row's outputs; dh and dg come from the separately pinned backward)."""
    M, d_in, d_out, r = 23, 70, 50, 96
    p = small(M, d_in, d_out, r, seed=85)
    GU, GV = oracle.sign_grads(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    dh, _, dg, _ = oracle.backward(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    SU = unpack_signs(p["bits_u"], d_out, r)
    SV = unpack_signs(p["bits_v"], d_in, r)
    h, g = p["h"].astype(np.float64), p["g"].astype(np.float64)
    assert oracle.rel_frobenius(np.sum(SU * GU, axis=1), h * dh) < 1e-12
    assert oracle.rel_frobenius(np.sum(SV * GV, axis=1), g * dg) < 1e-12


def test_sign_grads_accumulate_and_zero_dy():
    M, d_in, d_out, r = 9, 20, 12, 64
    p = small(M, d_in, d_out, r, seed=87)
    GU, GV = oracle.sign_grads(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    rng = np.random.default_rng(3)
    gu0, gv0 = rng.standard_normal(GU.shape), rng.standard_normal(GV.shape)
    GU2, GV2 = oracle.sign_grads(p["x"], p["dy"], p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"],
                                 gu0=gu0, gv0=gv0, accumulate=True)
    assert np.allclose(GU2, gu0 + GU, rtol=0, atol=1e-13) and np.allclose(GV2, gv0 + GV, rtol=0, atol=1e-13)
    Z = oracle.sign_grads(p["x"], np.zeros_like(p["dy"]), p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"])
    assert not np.any(Z[0]) and not np.any(Z[1])


# ----------------------------------------------------------- sum of squares --

def test_sumsq_closed_forms_and_non_finite():
    assert oracle.sumsq(np.array([3.0, 4.0])) == 25.0
    assert oracle.sumsq(np.ones(1000)) == 1000.0
    assert oracle.sumsq(np.zeros(7)) == 0.0
    n = 1001
    k = np.arange(1, n + 1, dtype=np.float64)
    assert oracle.sumsq(k) == n * (n + 1) * (2 * n + 1) / 6  # exact in f64 at this size
    assert oracle.sumsq(np.array([1.0, np.inf, 2.0])) == np.inf
    assert np.isnan(oracle.sumsq(np.array([1.0, np.nan])))
    assert np.isnan(oracle.sumsq(np.array([np.inf, -np.inf, np.nan])))


# ------------------------------------------------ the acceptance measure --
# rel = ||got - want||_F / max(||want||_F, 1e-15), the measure of test
# `blr_layer_matches_host` on the page (its `rel` closure). Every GPU parity
# check rests on it, so it is pinned by values that a dropped square root,
# a dropped floor or a swapped argument would change.

def test_rel_frobenius_closed_forms():
    w = np.array([[3.0, -4.0], [12.0, 0.0]])  # ||w|| = 13
    assert oracle.rel_frobenius(2 * w, w) == 1.0
    assert oracle.rel_frobenius(w, w) == 0.0
    assert oracle.rel_frobenius(np.zeros_like(w), w) == 1.0
    # got = w (1 + eps) with eps a power of two: every difference is exact,
    # so the measure is eps exactly (without the root it would be eps^2)
    for eps in (2.0 ** -1, 2.0 ** -10, 2.0 ** -20):
        assert oracle.rel_frobenius(w * (1 + eps), w) == eps
    # ||e|| = 2.5 against ||want|| = 5: 0.5 (0.25 without the root)
    assert oracle.rel_frobenius(np.array([4.5, 6.0]), np.array([3.0, 4.0])) == 0.5
    # asymmetric: the norm of the second argument is the denominator
    assert oracle.rel_frobenius(np.array([3.0, 4.0]), np.array([6.0, 8.0])) == 0.5
    assert oracle.rel_frobenius(np.array([6.0, 8.0]), np.array([3.0, 4.0])) == 1.0
    # f32 inputs are promoted exactly
    assert oracle.rel_frobenius(np.float32([4.5, 6.0]), np.float32([3.0, 4.0])) == 0.5


def test_rel_frobenius_floor_for_a_zero_reference():
    """A zero reference divides by the floor 1e-15 (the page's
    max(norm, 1e-15)), so a got of norm 5e-16 reads 0.5 and an exact zero 0."""
    z = np.zeros(2)
    assert oracle.rel_frobenius(z, z) == 0.0
    assert abs(oracle.rel_frobenius(np.array([3e-16, 4e-16]), z) - 0.5) < 1e-12
    assert abs(oracle.rel_frobenius(np.array([3e-13, 4e-13]), z) - 500.0) < 1e-9
    # the floor only acts below it
    assert abs(oracle.rel_frobenius(np.array([3e-15, 4e-15]), np.array([6e-15, 8e-15])) - 0.5) < 1e-12


def test_rel_frobenius_non_finite_fails_the_bar():
    w = np.array([1.0, 2.0])
    assert not oracle.rel_frobenius(np.array([np.nan, 2.0]), w) <= 3e-3
    assert not oracle.rel_frobenius(np.array([np.inf, 2.0]), w) <= 3e-3


# ----------------------------------------------------------- plane_linear --

def test_f16_decode_matches_numpy_float16():
    pats = np.array([0x3C00, 0xBC00, 0x7BFF, 0x0001, 0x03FF, 0x0400, 0x8001, 0x0000, 0x8000, 0x7C00, 0xFC00,
                     0x3555, 0x4248], dtype=np.uint16)
    want = pats.view(np.float16).astype(np.float64)
    got = oracle.f16_decode(pats)
    assert np.array_equal(got, want)
    assert np.isnan(oracle.f16_decode(np.array([0x7E00], np.uint16))[0])
    allp = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    a, b = oracle.f16_decode(allp), allp.view(np.float16).astype(np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(a[fin], b[fin]) and np.array_equal(np.isnan(a), np.isnan(b))


def test_plane_linear_identity_and_dense():
    rng = np.random.default_rng(91)
    k = 48
    x = rng.standard_normal((7, k))
    eye = np.eye(k).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.plane_linear(x, eye), x)
    plane = rng.standard_normal((30, k)).astype(np.float16)
    want = x @ plane.astype(np.float64).T
    assert oracle.rel_frobenius(oracle.plane_linear(x, plane.view(np.uint16)), want) < 1e-14


# ------------------------------------------------------------- paths --

def _paths(M, d_in, d_out, r, P, seed):
    return synth.custom_paths(M, d_in, d_out, r, P, seed, dy_sigma=1.0, l_hi=1.0)


def _path(d, p):
    return {"x": d["x"], "dy": d["dy"], **{k: d[k][p] for k in ("bits_u", "bits_v", "h", "l", "g")}}


@pytest.mark.parametrize("M,d_in,d_out,r,P", [(5, 7, 6, 40, 2), (33, 16, 24, 64, 3)])
def test_paths_forward_matches_dense_sum(M, d_in, d_out, r, P):
    """y = x . (sum_p W_p)^T with each W_p materialised from numpy's bit
    unpacking; the tape is the paths' a side by side."""
    d = _paths(M, d_in, d_out, r, P, 700 + M)
    y, a = oracle.forward_paths(d["x"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    W = sum(dense_w(_path(d, p)) for p in range(P))
    assert oracle.rel_frobenius(y, d["x"].astype(np.float64) @ W.T) < 1e-12
    assert a.shape == (M, P * r)
    for p in range(P):
        SV = unpack_signs(d["bits_v"][p], d_in, r)
        ap = (d["x"].astype(np.float64) * d["g"][p].astype(np.float64)) @ SV
        assert oracle.rel_frobenius(a[:, p * r:(p + 1) * r], ap) < 1e-12


def test_paths_backward_central_differences_and_dense():
    """Each path's dh, dl, dg are exact central differences of
    L = sum(dy . y) of the whole layer (y is linear in every parameter);
    dx = dy . sum_p W_p."""
    M, d_in, d_out, r, P = 3, 5, 4, 33, 2
    d = _paths(M, d_in, d_out, r, P, 711)
    dh, dl, dg, dx = oracle.backward_paths(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    W = sum(dense_w(_path(d, p)) for p in range(P))
    assert oracle.rel_frobenius(dx, d["dy"].astype(np.float64) @ W) < 1e-12

    def L(**kw):
        q = {k: d[k].astype(np.float64).copy() for k in ("h", "l", "g")}
        q.update(kw)
        y, _ = oracle.forward_paths(d["x"], d["bits_u"], d["bits_v"], q["h"], q["l"], q["g"])
        return float(np.sum(d["dy"].astype(np.float64) * y))

    eps = 0.25
    for name, got in (("h", dh), ("l", dl), ("g", dg)):
        base = d[name].astype(np.float64)
        fd = np.empty(base.shape)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += eps
            minus[idx] -= eps
            fd[idx] = (L(**{name: plus}) - L(**{name: minus})) / (2 * eps)
        assert oracle.rel_frobenius(got, fd) < 1e-10, name


def test_paths_identical_paths_and_permutation():
    """Two copies of one path double y and dx and repeat its own dh, dl, dg;
    reordering the paths reorders the per-path gradients and leaves y, dx."""
    M, d_in, d_out, r = 9, 12, 10, 40
    one = _paths(M, d_in, d_out, r, 1, 720)
    two = {k: (np.concatenate([v, v]) if k in ("bits_u", "bits_v", "h", "l", "g") else v) for k, v in one.items()}
    y1, _ = oracle.forward_paths(one["x"], one["bits_u"], one["bits_v"], one["h"], one["l"], one["g"])
    y2, _ = oracle.forward_paths(two["x"], two["bits_u"], two["bits_v"], two["h"], two["l"], two["g"])
    assert np.allclose(y2, 2 * y1, rtol=0, atol=1e-12 * np.abs(y1).max())
    g1 = oracle.backward_paths(one["x"], one["dy"], one["bits_u"], one["bits_v"], one["h"], one["l"], one["g"])
    g2 = oracle.backward_paths(two["x"], two["dy"], two["bits_u"], two["bits_v"], two["h"], two["l"], two["g"])
    for a, b in zip(g1[:3], g2[:3]):
        assert np.array_equal(b[0], a[0]) and np.array_equal(b[1], a[0])
    assert np.allclose(g2[3], 2 * g1[3], rtol=0, atol=1e-12 * np.abs(g1[3]).max())
    d = _paths(M, d_in, d_out, r, 3, 730)
    perm = [2, 0, 1]
    q = {k: (d[k][perm] if k in ("bits_u", "bits_v", "h", "l", "g") else d[k]) for k in d}
    ya, _ = oracle.forward_paths(d["x"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    yb, _ = oracle.forward_paths(q["x"], q["bits_u"], q["bits_v"], q["h"], q["l"], q["g"])
    assert oracle.rel_frobenius(yb, ya) < 1e-13
    ga = oracle.backward_paths(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    gb = oracle.backward_paths(q["x"], q["dy"], q["bits_u"], q["bits_v"], q["h"], q["l"], q["g"])
    for a, b in zip(ga[:3], gb[:3]):
        assert np.array_equal(b, a[perm])
    assert oracle.rel_frobenius(gb[3], ga[3]) < 1e-13


def test_paths_sign_grads_are_each_paths_own():
    """A path's sign gradients do not depend on the other paths (y is a sum
    over paths); they pass the relaxed flip identity of a single path."""
    M, d_in, d_out, r, P = 6, 9, 7, 40, 2
    d = _paths(M, d_in, d_out, r, P, 740)
    gu, gv = oracle.sign_grads_paths(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    for p in range(P):
        su, sv = oracle.sign_grads(d["x"], d["dy"], d["bits_u"][p], d["bits_v"][p], d["h"][p], d["l"][p], d["g"][p])
        assert np.array_equal(gu[p], su) and np.array_equal(gv[p], sv)
    # Euler: sum_k S_U . G_U = h . dh per path, against the paths' backward
    dh, _, dg, _ = oracle.backward_paths(d["x"], d["dy"], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
    for p in range(P):
        SU = unpack_signs(d["bits_u"][p], d_out, r)
        assert oracle.rel_frobenius((SU * gu[p]).sum(1), d["h"][p] * dh[p]) < 1e-12
