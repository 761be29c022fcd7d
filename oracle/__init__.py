"""f64 CPU oracle of the `blr` layer (ctypes over oracle/blr_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the product path never does. It shares no code
with the HIP library and imports nothing from it.

Source: the cortiq-engine page "src/gpu_wgpu/train_mm.rs" (0.8.21): module
doc block (layer and equations), `expand` shader (bit convention),
`blr_forward` / `blr_backward` (overwrite/accumulate rules); the acceptance
measure `rel_frobenius` is the relative error of the page's layer test.

Every function takes numpy arrays; floating inputs are promoted to f64
exactly. Every function here is pinned by tests/test_oracle.py against
facts outside the oracle: numpy's own bit unpacking, dense materialisation
of the layer matrix, rank-one closed forms, a hand-worked example, exact
central differences, Euler identities and the sign-flip identity.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "blr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_threads.restype = i32
        lib.oracle_decode_signs.argtypes = [p, i64, i64, p]
        lib.oracle_expand_planes.argtypes = [p, i64, i64, p, p]
        lib.oracle_blr_forward.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, i32, p, p]
        lib.oracle_blr_forward.restype = i32
        lib.oracle_blr_backward.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, p, p, i32]
        lib.oracle_blr_backward.restype = i32
        lib.oracle_blr_sign_grads.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, i32]
        lib.oracle_blr_sign_grads.restype = i32
        lib.oracle_f16_decode.argtypes = [p, i64, p]
        lib.oracle_plane_linear.argtypes = [i64, i64, i64, p, p, p]
        lib.oracle_plane_linear.restype = i32
        lib.oracle_sumsq.argtypes = [p, i64]
        lib.oracle_sumsq.restype = ctypes.c_double
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _u32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint32:
        raise TypeError("bitmaps must be uint32")
    return a


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def threads() -> int:
    return int(_load().oracle_threads())


def decode_signs(bits, rows: int, r: int) -> np.ndarray:
    """S[rows][r] of +-1.0 (`expand` shader convention)."""
    bits = _u32(bits)
    assert bits.size == rows * ((r + 31) // 32)
    S = np.empty((rows, r), dtype=np.float64)
    _load().oracle_decode_signs(_ptr(bits), rows, r, _ptr(S))
    return S


def expand_planes(bits, rows: int, r: int) -> tuple[np.ndarray, np.ndarray]:
    """The f16 bit patterns PL[rows][r] and PLT[r][rows] (uint16)."""
    bits = _u32(bits)
    assert bits.size == rows * ((r + 31) // 32)
    pl = np.empty((rows, r), dtype=np.uint16)
    plt = np.empty((r, rows), dtype=np.uint16)
    _load().oracle_expand_planes(_ptr(bits), rows, r, _ptr(pl), _ptr(plt))
    return pl, plt


def forward(x, bits_u, bits_v, h, l, g, y0=None, accumulate: bool = False, tape: bool = True):
    """Returns (y, a, c) in f64; a, c are None when tape is False."""
    x = _f64(x)
    M, d_in = x.shape
    h, l, g = _f64(h), _f64(l), _f64(g)
    d_out, r = h.size, l.size
    assert g.size == d_in
    bits_u, bits_v = _u32(bits_u), _u32(bits_v)
    W = (r + 31) // 32
    assert bits_u.size == d_out * W and bits_v.size == d_in * W
    y = np.zeros((M, d_out)) if y0 is None else _f64(y0).copy()
    a = np.empty((M, r)) if tape else None
    c = np.empty((M, d_out)) if tape else None
    rc = _load().oracle_blr_forward(M, d_in, d_out, r, _ptr(x), _ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l),
                                    _ptr(g), _ptr(y), int(bool(accumulate)), _ptr(a), _ptr(c))
    if rc != 0:
        raise MemoryError("oracle forward: out of memory")
    return y, a, c


def backward(x, dy, bits_u, bits_v, h, l, g, dh0=None, dl0=None, dg0=None, dx0=None, accumulate_dx: bool = False):
    """Returns (dh, dl, dg, dx) in f64. dh/dl/dg start from dh0/dl0/dg0
    (zeros by default) and accumulate; dx is overwritten unless
    accumulate_dx, then it adds to dx0."""
    x, dy = _f64(x), _f64(dy)
    M, d_in = x.shape
    h, l, g = _f64(h), _f64(l), _f64(g)
    d_out, r = h.size, l.size
    assert dy.shape == (M, d_out) and g.size == d_in
    bits_u, bits_v = _u32(bits_u), _u32(bits_v)
    W = (r + 31) // 32
    assert bits_u.size == d_out * W and bits_v.size == d_in * W
    dh = np.zeros(d_out) if dh0 is None else _f64(dh0).copy()
    dl = np.zeros(r) if dl0 is None else _f64(dl0).copy()
    dg = np.zeros(d_in) if dg0 is None else _f64(dg0).copy()
    dx = np.zeros((M, d_in)) if dx0 is None else _f64(dx0).copy()
    rc = _load().oracle_blr_backward(M, d_in, d_out, r, _ptr(x), _ptr(dy), _ptr(bits_u), _ptr(bits_v), _ptr(h),
                                     _ptr(l), _ptr(g), _ptr(dh), _ptr(dl), _ptr(dg), _ptr(dx),
                                     int(bool(accumulate_dx)))
    if rc != 0:
        raise MemoryError("oracle backward: out of memory")
    return dh, dl, dg, dx


def sign_grads(x, dy, bits_u, bits_v, h, l, g, gu0=None, gv0=None, accumulate: bool = False):
    """Returns (G_U [d_out][r], G_V [d_in][r]) in f64: the gradients of
    sum(dy * y) with respect to the entries of S_U and S_V taken as real
    numbers. Without accumulate they are overwritten, else added to gu0/gv0."""
    x, dy = _f64(x), _f64(dy)
    M, d_in = x.shape
    h, l, g = _f64(h), _f64(l), _f64(g)
    d_out, r = h.size, l.size
    assert dy.shape == (M, d_out) and g.size == d_in
    bits_u, bits_v = _u32(bits_u), _u32(bits_v)
    W = (r + 31) // 32
    assert bits_u.size == d_out * W and bits_v.size == d_in * W
    gu = np.zeros((d_out, r)) if gu0 is None else _f64(gu0).copy()
    gv = np.zeros((d_in, r)) if gv0 is None else _f64(gv0).copy()
    rc = _load().oracle_blr_sign_grads(M, d_in, d_out, r, _ptr(x), _ptr(dy), _ptr(bits_u), _ptr(bits_v), _ptr(h),
                                       _ptr(l), _ptr(g), _ptr(gu), _ptr(gv), int(bool(accumulate)))
    if rc != 0:
        raise MemoryError("oracle sign gradients: out of memory")
    return gu, gv


def forward_paths(x, bits_u, bits_v, h, l, g, y0=None, accumulate: bool = False):
    """A layer of P paths (page: `blr_forward` over a layer's paths: the
    first path overwrites y unless accumulating, every later path adds):
    y = sum_p h_p . c_p with path p's operands bits_u[p], bits_v[p], h[p],
    l[p], g[p]. Returns (y, a) in f64, a [M][P r] (the paths' a side by
    side)."""
    h = _f64(h)
    P = h.shape[0]
    y, tapes = None if y0 is None else _f64(y0), []
    for p in range(P):
        y, a, _ = forward(x, bits_u[p], bits_v[p], h[p], l[p], g[p], y0=y, accumulate=accumulate or p > 0)
        tapes.append(a)
    return y, np.concatenate(tapes, axis=1)


def backward_paths(x, dy, bits_u, bits_v, h, l, g, dx0=None, accumulate_dx: bool = False):
    """Backward of a layer of P paths (page: `blr_backward` over the paths,
    dx overwritten by the first path unless accumulating, added by later
    ones): dh [P][d_out], dl [P][r], dg [P][d_in] from zero, and
    dx = sum_p g_p . dx'_p. Returns (dh, dl, dg, dx) in f64."""
    h = _f64(h)
    P = h.shape[0]
    dx, dhs, dls, dgs = None if dx0 is None else _f64(dx0), [], [], []
    for p in range(P):
        dh, dl, dg, dx = backward(x, dy, bits_u[p], bits_v[p], h[p], l[p], g[p], dx0=dx,
                                  accumulate_dx=accumulate_dx or p > 0)
        dhs.append(dh)
        dls.append(dl)
        dgs.append(dg)
    return np.stack(dhs), np.stack(dls), np.stack(dgs), dx


def sign_grads_paths(x, dy, bits_u, bits_v, h, l, g):
    """The sign gradients of every path of a layer: (G_U [P][d_out][r],
    G_V [P][d_in][r]) in f64 (each path's, as in sign_grads: y is linear in
    each path's signs, so the other paths do not enter)."""
    h = _f64(h)
    gus, gvs = [], []
    for p in range(h.shape[0]):
        gu, gv = sign_grads(x, dy, bits_u[p], bits_v[p], h[p], l[p], g[p])
        gus.append(gu)
        gvs.append(gv)
    return np.stack(gus), np.stack(gvs)


def f16_decode(bits) -> np.ndarray:
    """f64 values of IEEE binary16 bit patterns (uint16)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_f16_decode(_ptr(bits), bits.size, _ptr(out))
    return out


def plane_linear(x, plane_bits) -> np.ndarray:
    """y [M][n] = x [M][k] times the transpose of the f16 plane [n][k] (uint16
    bit patterns), in f64 (the page's `plane_linear`; its scale cancels)."""
    x = _f64(x)
    M, k = x.shape
    plane_bits = np.ascontiguousarray(plane_bits, dtype=np.uint16)
    n = plane_bits.shape[0]
    assert plane_bits.shape == (n, k)
    y = np.empty((M, n))
    if _load().oracle_plane_linear(M, n, k, _ptr(x), _ptr(plane_bits), _ptr(y)) != 0:
        raise MemoryError("oracle plane_linear: out of memory")
    return y


def sumsq(a) -> float:
    """sum(a**2) in f64, in index order; non-finite values propagate."""
    a = _f64(a).ravel()
    return float(_load().oracle_sumsq(_ptr(a), a.size))


def rel_frobenius(got, want) -> float:
    """Relative Frobenius error: ||got - want|| / max(||want||, 1e-15), the
    acceptance measure of test `blr_layer_matches_host`."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    num = float(np.sum((got - want) ** 2))
    den = max(float(np.sum(want * want)), 1e-30)
    return (num / den) ** 0.5
