"""C ABI checks that need no GPU: the library loads, exports every function
include/blr.h declares, sizes workspaces, and rejects bad arguments before
touching the device (nothing is launched on any error path tested here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import binary_rank_linear_amd as blr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blr.h")

BLR_OK, E_NULL, E_SHAPE, E_SCALE, E_WS, E_DEV, E_HIP, E_ALIGN, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(blr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("blr_forward", "blr_backward", "blr_expand_signs", "blr_workspace_bytes", "blr_status_string",
              "blr_device_supported"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = blr.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", blr.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (blr_[a-z_]+)\b", out))
    assert set(declared_functions()) <= exported


def test_library_is_gfx950_only():
    """The offload bundle of our own build holds code for gfx950 only."""
    data = open(blr.LIB_PATH, "rb").read()
    arches = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", data))
    assert arches == {b"gfx950"}, arches


def test_status_strings():
    for s in (BLR_OK, E_NULL, E_SHAPE, E_SCALE, E_WS, E_DEV, E_HIP, E_ALIGN, E_SCRATCH):
        assert blr.status_string(s) and blr.status_string(s) != "unknown status"
    assert blr.status_string(-99) == "unknown status"


def test_workspace_bytes():
    assert blr.blr_workspace_bytes(8192, 4096, 4096, 512) > 0
    # transposed bitmap [r][max(d)/32] words + db [M][r] f32 + column partials
    n = blr.blr_workspace_bytes(128, 256, 256, 128)
    assert n >= 4 * 128 * (256 // 32) + 4 * 128 * 128
    assert n % 256 == 0
    assert blr.blr_workspace_bytes(30000, 5120, 17408, 2048) >= 4 * 30000 * 2048
    for bad in [(0, 256, 256, 128), (128, 200, 256, 128), (128, 256, 100, 128), (128, 256, 256, 64), (-1, 256, 256, 128),
                (1 << 21, 1 << 10, 1 << 10, 128)]:  # an operand of 8 GiB: beyond 32-bit byte offsets
        assert blr.blr_workspace_bytes(*bad) == 0


class Fake:
    """Aligned host buffers standing in for device pointers: every call
    below fails validation before any device work, so they are never
    dereferenced."""

    def __init__(self):
        self.keep = []

    def __call__(self, nbytes=256, offset=0):
        a = np.zeros(nbytes + 64, np.uint8)
        self.keep.append(a)
        base = a.ctypes.data
        return ctypes.c_void_p(((base + 15) // 16) * 16 + offset)


def fwd(lib, M, d_in, d_out, r, ptrs, ws_bytes=None):
    ws_bytes = blr.blr_workspace_bytes(M, d_in, d_out, r) if ws_bytes is None else ws_bytes
    return lib.blr_forward(M, d_in, d_out, r, ptrs["x"], ptrs["bu"], ptrs["bv"], ptrs["h"], ptrs["l"], ptrs["g"],
                           ptrs["y"], 0, ptrs["ta"], ptrs["tc"], ptrs["ws"], ws_bytes, None)


def bwd(lib, M, d_in, d_out, r, ptrs, gscale=1024.0, ws_bytes=None):
    ws_bytes = blr.blr_workspace_bytes(M, d_in, d_out, r) if ws_bytes is None else ws_bytes
    return lib.blr_backward(M, d_in, d_out, r, ptrs["x"], ptrs["dy"], ptrs["bu"], ptrs["bv"], ptrs["h"],
                            ptrs["l"], ptrs["g"], ptrs["ta"], ptrs["tc"], ctypes.c_float(gscale), ptrs["dh"],
                            ptrs["dl"], ptrs["dg"], ptrs["dx"], 0, ptrs["ws"], ws_bytes, None)


KEYS = ["x", "dy", "bu", "bv", "h", "l", "g", "y", "ta", "tc", "dh", "dl", "dg", "dx", "ws"]


@pytest.fixture
def ptrs():
    f = Fake()
    d = {k: f() for k in KEYS}
    d["_fake"] = f
    return d


def test_forward_rejects_null(ptrs):
    lib = blr.load()
    for k in ["x", "bu", "bv", "h", "l", "g", "y", "ta"]:
        p = dict(ptrs)
        p[k] = None
        assert fwd(lib, 128, 256, 256, 128, p) == E_NULL, k


def test_backward_rejects_null(ptrs):
    lib = blr.load()
    for k in ["x", "dy", "bu", "bv", "h", "l", "g", "ta", "dh", "dl", "dg", "dx"]:
        p = dict(ptrs)
        p[k] = None
        assert bwd(lib, 128, 256, 256, 128, p) == E_NULL, k


@pytest.mark.parametrize("shape", [(0, 256, 256, 128), (128, 200, 256, 128), (128, 256, 300, 128),
                                   (128, 256, 256, 96), (128, 256, 256, 0), (-5, 256, 256, 128),
                                   (128, 0, 256, 128)])
def test_rejects_bad_shapes(ptrs, shape):
    lib = blr.load()
    assert fwd(lib, *shape, ptrs, ws_bytes=1 << 40) == E_SHAPE
    assert bwd(lib, *shape, ptrs, ws_bytes=1 << 40) == E_SHAPE


@pytest.mark.parametrize("M,d_in,d_out,r", [(65535, 16384, 128, 128), (65535, 128, 16384, 128),
                                           (32767, 128, 128, 32768)], ids=["x_dx", "y_dy", "db"])
def test_operand_size_edge(ptrs, M, d_in, d_out, r):
    """The kernels address every operand with 32-bit byte offsets: a shape
    whose largest operand (x and dx, y and dy, or the db workspace) is one
    token short of 4 GiB is accepted; one more token, exactly 4 GiB, is
    rejected before any device work."""
    lib = blr.load()
    assert blr.blr_workspace_bytes(M, d_in, d_out, r) > 0
    assert blr.blr_workspace_bytes(M + 1, d_in, d_out, r) == 0
    assert fwd(lib, M + 1, d_in, d_out, r, ptrs, ws_bytes=1 << 40) == E_SHAPE
    assert bwd(lib, M + 1, d_in, d_out, r, ptrs, ws_bytes=1 << 40) == E_SHAPE


@pytest.mark.parametrize("gs", [0.0, -1024.0, 3.0, 1000.0, float("inf"), float("nan"), 1.5])
def test_backward_rejects_bad_gscale(ptrs, gs):
    assert bwd(blr.load(), 128, 256, 256, 128, ptrs, gscale=gs) == E_SCALE


def test_rejects_small_workspace(ptrs):
    lib = blr.load()
    need = blr.blr_workspace_bytes(128, 256, 256, 128)
    assert fwd(lib, 128, 256, 256, 128, ptrs, ws_bytes=need - 1) == E_WS
    assert bwd(lib, 128, 256, 256, 128, ptrs, ws_bytes=need - 1) == E_WS
    p = dict(ptrs)
    p["ws"] = None
    assert fwd(lib, 128, 256, 256, 128, p) == E_WS


def test_rejects_misaligned(ptrs):
    lib = blr.load()
    f = ptrs["_fake"]
    for k in ["x", "y", "ta", "h"]:
        p = dict(ptrs)
        p[k] = f(offset=4)
        assert fwd(lib, 128, 256, 256, 128, p) == E_ALIGN, k
    p = dict(ptrs)
    p["dx"] = f(offset=8)
    assert bwd(lib, 128, 256, 256, 128, p) == E_ALIGN
    # bitmaps are read as 16-byte groups of 4 words
    for k in ["bu", "bv"]:
        p = dict(ptrs)
        p[k] = f(offset=4)
        assert fwd(lib, 128, 256, 256, 128, p) == E_ALIGN, k
        assert bwd(lib, 128, 256, 256, 128, p) == E_ALIGN, k


def test_expand_rejects_bad_arguments(ptrs):
    lib = blr.load()
    f = ptrs["_fake"]
    assert lib.blr_expand_signs(None, 4, 32, f(), f(), None) == E_NULL
    assert lib.blr_expand_signs(f(), 4, 32, None, None, None) == E_NULL
    assert lib.blr_expand_signs(f(), 0, 32, f(), None, None) == E_SHAPE
    assert lib.blr_expand_signs(f(), 4, 0, None, f(), None) == E_SHAPE
    assert lib.blr_expand_signs(f(), 4, 32, f(offset=2), None, None) == E_ALIGN


def bwd_signs(lib, M, d_in, d_out, r, ptrs, gscale=1024.0):
    ws_bytes = blr.blr_workspace_bytes(M, d_in, d_out, r)
    return lib.blr_backward_signs(M, d_in, d_out, r, ptrs["x"], ptrs["dy"], ptrs["bu"], ptrs["bv"], ptrs["h"],
                                  ptrs["l"], ptrs["g"], ptrs["ta"], ptrs["tc"], ctypes.c_float(gscale), ptrs["dh"],
                                  ptrs["dl"], ptrs["dg"], ptrs["dx"], 0, ptrs["gu"], ptrs["gv"], 0, ptrs["ws"],
                                  ws_bytes, None)


def test_backward_signs_rejects_bad_arguments(ptrs):
    lib = blr.load()
    f = ptrs["_fake"]
    p = dict(ptrs)
    p["gu"], p["gv"] = f(), f()
    for k in ["gu", "gv", "x", "dy", "ta"]:
        q = dict(p)
        q[k] = None
        assert bwd_signs(lib, 128, 256, 256, 128, q) == E_NULL, k
    for k in ["gu", "gv"]:
        q = dict(p)
        q[k] = f(offset=4)
        assert bwd_signs(lib, 128, 256, 256, 128, q) == E_ALIGN, k
    assert bwd_signs(lib, 128, 200, 256, 128, p) == E_SHAPE
    assert bwd_signs(lib, 128, 256, 256, 128, p, gscale=3.0) == E_SCALE


def test_sumsq_rejects_bad_arguments(ptrs):
    lib = blr.load()
    f = ptrs["_fake"]
    assert lib.blr_sumsq(None, 16, f(), 4, None) == E_NULL
    assert lib.blr_sumsq(f(), 16, None, 4, None) == E_NULL
    assert lib.blr_sumsq(f(), 0, f(), 4, None) == E_SHAPE
    assert lib.blr_sumsq(f(), 16, f(), 0, None) == E_SHAPE
    assert lib.blr_sumsq(f(), 16, f(), 1025, None) == E_SHAPE
    assert lib.blr_sumsq(f(offset=4), 16, f(), 4, None) == E_ALIGN


def test_next_gscale_doubles_on_success_and_halves_on_overflow():
    assert blr.next_gscale(1024.0, True) == 2048.0
    assert blr.next_gscale(1024.0, False) == 512.0
    assert blr.next_gscale(2.0 ** 24, True) == 2.0 ** 24
    assert blr.next_gscale(1.0, False) == 1.0
    g = 2.0 ** 10
    for finite in (True, False, False, True):
        g = blr.next_gscale(g, finite)
        m, e = np.frexp(g)
        assert m == 0.5  # stays a power of two


def test_plane_linear_rejects_bad_arguments(ptrs):
    lib = blr.load()
    f = ptrs["_fake"]
    good = (128, 256, 128, f(), f(), f(), ctypes.c_float(1.0), None)
    assert lib.blr_plane_linear(128, 256, 128, None, f(), f(), ctypes.c_float(1.0), None) == E_NULL
    assert lib.blr_plane_linear(128, 200, 128, f(), f(), f(), ctypes.c_float(1.0), None) == E_SHAPE
    assert lib.blr_plane_linear(0, 256, 128, f(), f(), f(), ctypes.c_float(1.0), None) == E_SHAPE
    assert lib.blr_plane_linear(128, 256, 128, f(), f(), f(), ctypes.c_float(3.0), None) == E_SCALE
    assert lib.blr_plane_linear(128, 256, 128, f(offset=4), f(), f(), ctypes.c_float(1.0), None) == E_ALIGN
    assert len(good) == 8


def test_paths_workspace_and_rejects(ptrs):
    lib = blr.load()
    one = blr.blr_workspace_bytes(256, 256, 256, 128)
    assert blr.blr_workspace_bytes_paths(256, 256, 256, 128, 1) == one
    assert blr.blr_workspace_bytes_paths(256, 256, 256, 128, 3) > one
    for bad in (0, 5, -1):
        assert blr.blr_workspace_bytes_paths(256, 256, 256, 128, bad) == 0
    f = ptrs["_fake"]
    ws = 1 << 40

    def fwd_p(P, r=128, **kw):
        q = {k: f() for k in ("x", "bu", "bv", "h", "l", "g", "y", "ta")}
        q.update(kw)
        return lib.blr_forward_paths(128, 256, 256, r, P, q["x"], q["bu"], q["bv"], q["h"], q["l"], q["g"], q["y"], 0,
                                     q["ta"], f(), ws, None)

    assert fwd_p(5) == E_SHAPE
    assert fwd_p(0) == E_SHAPE
    assert fwd_p(2, r=96) == E_SHAPE
    assert fwd_p(2, x=None) == E_NULL
    assert fwd_p(2, bu=f(offset=4)) == E_ALIGN
    q = {k: f() for k in KEYS}
    assert lib.blr_backward_paths(128, 256, 256, 128, 5, q["x"], q["dy"], q["bu"], q["bv"], q["h"], q["l"], q["g"],
                                  q["ta"], ctypes.c_float(1024.0), q["dh"], q["dl"], q["dg"], q["dx"], 0, None, None,
                                  0, q["ws"], ws, None) == E_SHAPE
    assert lib.blr_backward_paths(128, 256, 256, 128, 2, q["x"], q["dy"], q["bu"], q["bv"], q["h"], q["l"], q["g"],
                                  q["ta"], ctypes.c_float(3.0), q["dh"], q["dl"], q["dg"], q["dx"], 0, None, None,
                                  0, q["ws"], ws, None) == E_SCALE
    assert lib.blr_backward_paths(128, 256, 256, 128, 2, q["x"], q["dy"], q["bu"], q["bv"], q["h"], q["l"], q["g"],
                                  q["ta"], ctypes.c_float(1024.0), q["dh"], q["dl"], q["dg"], q["dx"], 0, f(), None,
                                  0, q["ws"], ws, None) == E_NULL


def fwd_noalloc(lib, M, d_in, d_out, r, ptrs):
    return lib.blr_forward_noalloc(M, d_in, d_out, r, ptrs["x"], ptrs["bu"], ptrs["bv"], ptrs["h"], ptrs["l"],
                                   ptrs["g"], ptrs["y"], 0, ptrs["ta"], ptrs["tc"], None)


def test_forward_noalloc_rejects_before_any_device_work(ptrs):
    """The allocation-free forward validates as blr_forward does, and rejects
    sizes whose transposed bitmap (r * d_in / 8 bytes) exceeds its scratch
    with its own status, before touching the device."""
    lib = blr.load()
    for k in ["x", "bu", "bv", "h", "l", "g", "y", "ta"]:
        p = dict(ptrs)
        p[k] = None
        assert fwd_noalloc(lib, 128, 256, 256, 128, p) == E_NULL, k
    for shape in [(0, 256, 256, 128), (128, 200, 256, 128), (128, 256, 256, 100)]:
        assert fwd_noalloc(lib, *shape, ptrs) == E_SHAPE, shape
    p = dict(ptrs)
    p["x"] = ptrs["_fake"](256, offset=4)
    assert fwd_noalloc(lib, 128, 256, 256, 128, p) == E_ALIGN
    # r * d_in / 8 one step of d_in past the scratch (2048 * 16384 / 8 is
    # exactly its size); sizes that pass every check are not called here,
    # since these fake pointers must never reach a launch
    assert 2048 * 16384 // 8 == blr.NOALLOC_SCRATCH_BYTES
    assert fwd_noalloc(lib, 64, 16384 + 128, 256, 2048, ptrs) == E_SCRATCH
    assert fwd_noalloc(lib, 64, 128, 256, 2048 * 128 + 128, ptrs) == E_SCRATCH
    assert "scratch" in blr.status_string(E_SCRATCH)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define BLR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == blr.NOALLOC_SCRATCH_BYTES
