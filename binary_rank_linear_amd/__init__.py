"""Python binding of libblr.so, the MI355X (gfx950) binary low-rank (`blr`)
linear layer (C ABI in include/blr.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI. PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or the device is not
gfx950, the calls raise.

The functions carry the C names: `blr_expand_signs`, `blr_forward`,
`blr_forward_noalloc`, `blr_backward`, `blr_backward_signs`, `blr_plane_linear`, `blr_sumsq`, `blr_workspace_bytes`,
plus the profiling calls; `all_finite` and `next_gscale` are the host side
of the finite check and the power-of-two loss scale.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblr.so")
_lib = None


class BlrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load():
    """Load libblr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m binary_rank_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, p, i32, f32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.blr_status_string.argtypes = [i32]
    lib.blr_status_string.restype = ctypes.c_char_p
    lib.blr_device_supported.argtypes = [i32]
    lib.blr_device_supported.restype = i32
    lib.blr_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.blr_workspace_bytes.restype = sz
    lib.blr_expand_signs.argtypes = [p, i64, i64, p, p, p]
    lib.blr_expand_signs.restype = i32
    lib.blr_forward.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, i32, p, p, p, sz, p]
    lib.blr_forward.restype = i32
    lib.blr_forward_noalloc.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, i32, p, p, p]
    lib.blr_forward_noalloc.restype = i32
    lib.blr_backward.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, f32, p, p, p, p, i32, p, sz, p]
    lib.blr_backward.restype = i32
    lib.blr_backward_signs.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, f32, p, p, p, p, i32, p, p, i32,
                                       p, sz, p]
    lib.blr_backward_signs.restype = i32
    lib.blr_workspace_bytes_paths.argtypes = [i64, i64, i64, i64, i64]
    lib.blr_workspace_bytes_paths.restype = sz
    lib.blr_forward_paths.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, p, p, i32, p, p, sz, p]
    lib.blr_forward_paths.restype = i32
    lib.blr_backward_paths.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p, f32, p, p, p, p, i32, p, p,
                                       i32, p, sz, p]
    lib.blr_backward_paths.restype = i32
    lib.blr_plane_linear.argtypes = [i64, i64, i64, p, p, p, f32, p]
    lib.blr_plane_linear.restype = i32
    lib.blr_sumsq.argtypes = [p, i64, p, i32, p]
    lib.blr_sumsq.restype = i32
    lib.blr_profile_enable.argtypes = [i32]
    lib.blr_profile_enable.restype = i32
    lib.blr_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i64),
                                     ctypes.POINTER(ctypes.c_double), i32]
    lib.blr_profile_read.restype = i32
    lib.blr_profile_reset.argtypes = []
    lib.blr_profile_reset.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().blr_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise BlrError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtypes, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _bits_dtypes():
    import torch
    return (torch.int32, getattr(torch, "uint32", torch.int32))


def device_supported(device: int = 0) -> bool:
    return bool(load().blr_device_supported(int(device)))


def blr_workspace_bytes(M: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().blr_workspace_bytes(M, d_in, d_out, r))


def workspace(M: int, d_in: int, d_out: int, r: int, device=None):
    import torch
    n = blr_workspace_bytes(M, d_in, d_out, r)
    if n == 0:
        raise BlrError(-2, "blr_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def blr_expand_signs(bits, rows: int, r: int, plane=True, plane_t=True, stream=None):
    """Expand a sign bitmap [rows][ceil(r/32)] into f16 planes. `plane` /
    `plane_t` are output tensors (f16 [rows][r] / [r][rows]), True to
    allocate, or None to skip. Returns (plane, plane_t)."""
    import torch
    W = (r + 31) // 32
    _need(bits, "bits", _bits_dtypes(), (rows, W))
    if plane is True:
        plane = torch.empty((rows, r), dtype=torch.float16, device=bits.device)
    if plane_t is True:
        plane_t = torch.empty((r, rows), dtype=torch.float16, device=bits.device)
    if plane is not None:
        _need(plane, "plane", (torch.float16, torch.int16), (rows, r))
    if plane_t is not None:
        _need(plane_t, "plane_t", (torch.float16, torch.int16), (r, rows))
    _check(load().blr_expand_signs(_ptr(bits), rows, r, _ptr(plane), _ptr(plane_t), _stream(stream)),
           "blr_expand_signs")
    return plane, plane_t


def blr_forward(x, bits_u, bits_v, h, l, g, *, y=None, accumulate_y=False, tape_a=None, tape_c=None,
                keep_c=False, ws=None, stream=None):
    """Forward of one path. Returns (y, tape_a, tape_c); outputs not given
    are allocated. y is overwritten unless accumulate_y. The c tape is kept
    only when tape_c is given or keep_c is set; otherwise tape_c is None and
    blr_backward recomputes c."""
    import torch
    f32 = (torch.float32,)
    M, d_in = _need(x, "x", f32).shape
    d_out, r = _need(h, "h", f32).shape[0], _need(l, "l", f32).shape[0]
    _need(g, "g", f32, (d_in,))
    W = (r + 31) // 32
    _need(bits_u, "bits_u", _bits_dtypes(), (d_out, W))
    _need(bits_v, "bits_v", _bits_dtypes(), (d_in, W))
    dev = x.device
    y = torch.empty((M, d_out), dtype=torch.float32, device=dev) if y is None else _need(y, "y", f32, (M, d_out))
    tape_a = torch.empty((M, r), dtype=torch.float32, device=dev) if tape_a is None else \
        _need(tape_a, "tape_a", f32, (M, r))
    if tape_c is None and keep_c:
        tape_c = torch.empty((M, d_out), dtype=torch.float32, device=dev)
    if tape_c is not None:
        _need(tape_c, "tape_c", f32, (M, d_out))
    if ws is None:
        ws = workspace(M, d_in, d_out, r, dev)
    _check(load().blr_forward(M, d_in, d_out, r, _ptr(x), _ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l), _ptr(g),
                              _ptr(y), int(bool(accumulate_y)), _ptr(tape_a), _ptr(tape_c), _ptr(ws), ws.numel(),
                              _stream(stream)), "blr_forward")
    return y, tape_a, tape_c


# bytes of the allocation-free forward's scratch (BLR_NOALLOC_SCRATCH_BYTES):
# it serves sizes with r * d_in / 8 up to this
NOALLOC_SCRATCH_BYTES = 4 << 20


def blr_forward_noalloc(x, bits_u, bits_v, h, l, g, y, tape_a, *, accumulate_y=False, tape_c=None, stream=None):
    """blr_forward without a workspace and without allocating: every output
    (y, tape_a, and tape_c if kept) is the caller's; the library's own
    per-GPU scratch holds the transposed bitmap. Calls that overlap on one
    GPU race. Returns (y, tape_a, tape_c)."""
    import torch
    f32 = (torch.float32,)
    M, d_in = _need(x, "x", f32).shape
    d_out, r = _need(h, "h", f32).shape[0], _need(l, "l", f32).shape[0]
    _need(g, "g", f32, (d_in,))
    W = (r + 31) // 32
    _need(bits_u, "bits_u", _bits_dtypes(), (d_out, W))
    _need(bits_v, "bits_v", _bits_dtypes(), (d_in, W))
    _need(y, "y", f32, (M, d_out))
    _need(tape_a, "tape_a", f32, (M, r))
    if tape_c is not None:
        _need(tape_c, "tape_c", f32, (M, d_out))
    _check(load().blr_forward_noalloc(M, d_in, d_out, r, _ptr(x), _ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l),
                                      _ptr(g), _ptr(y), int(bool(accumulate_y)), _ptr(tape_a), _ptr(tape_c),
                                      _stream(stream)), "blr_forward_noalloc")
    return y, tape_a, tape_c


def blr_backward(x, dy, bits_u, bits_v, h, l, g, tape_a, tape_c, gscale: float, *, dh=None, dl=None, dg=None,
                 dx=None, accumulate_dx=False, ws=None, stream=None):
    """Backward of one path. dh/dl/dg accumulate (allocated as zeros when not
    given); dx is overwritten unless accumulate_dx. tape_c is the forward's
    c tape, or None when the forward kept none. Returns (dh, dl, dg, dx)."""
    import torch
    f32 = (torch.float32,)
    M, d_in = _need(x, "x", f32).shape
    d_out, r = _need(h, "h", f32).shape[0], _need(l, "l", f32).shape[0]
    _need(g, "g", f32, (d_in,))
    _need(dy, "dy", f32, (M, d_out))
    W = (r + 31) // 32
    _need(bits_u, "bits_u", _bits_dtypes(), (d_out, W))
    _need(bits_v, "bits_v", _bits_dtypes(), (d_in, W))
    _need(tape_a, "tape_a", f32, (M, r))
    if tape_c is not None:
        _need(tape_c, "tape_c", f32, (M, d_out))
    dev = x.device
    dh = torch.zeros(d_out, dtype=torch.float32, device=dev) if dh is None else _need(dh, "dh", f32, (d_out,))
    dl = torch.zeros(r, dtype=torch.float32, device=dev) if dl is None else _need(dl, "dl", f32, (r,))
    dg = torch.zeros(d_in, dtype=torch.float32, device=dev) if dg is None else _need(dg, "dg", f32, (d_in,))
    dx = torch.empty((M, d_in), dtype=torch.float32, device=dev) if dx is None else _need(dx, "dx", f32, (M, d_in))
    if ws is None:
        ws = workspace(M, d_in, d_out, r, dev)
    _check(load().blr_backward(M, d_in, d_out, r, _ptr(x), _ptr(dy), _ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l),
                               _ptr(g), _ptr(tape_a), _ptr(tape_c), ctypes.c_float(gscale), _ptr(dh), _ptr(dl),
                               _ptr(dg), _ptr(dx), int(bool(accumulate_dx)), _ptr(ws), ws.numel(), _stream(stream)),
           "blr_backward")
    return dh, dl, dg, dx


def blr_backward_signs(x, dy, bits_u, bits_v, h, l, g, tape_a, tape_c, gscale: float, *, dh=None, dl=None, dg=None,
                       dx=None, accumulate_dx=False, grad_u=None, grad_v=None, accumulate_signs=False, ws=None,
                       stream=None):
    """blr_backward plus the sign gradients G_U [d_out][r] and G_V [d_in][r]
    (allocated when not given; overwritten unless accumulate_signs).
    Returns (dh, dl, dg, dx, grad_u, grad_v)."""
    import torch
    f32 = (torch.float32,)
    M, d_in = _need(x, "x", f32).shape
    d_out, r = _need(h, "h", f32).shape[0], _need(l, "l", f32).shape[0]
    _need(g, "g", f32, (d_in,))
    _need(dy, "dy", f32, (M, d_out))
    W = (r + 31) // 32
    _need(bits_u, "bits_u", _bits_dtypes(), (d_out, W))
    _need(bits_v, "bits_v", _bits_dtypes(), (d_in, W))
    _need(tape_a, "tape_a", f32, (M, r))
    if tape_c is not None:
        _need(tape_c, "tape_c", f32, (M, d_out))
    dev = x.device
    dh = torch.zeros(d_out, dtype=torch.float32, device=dev) if dh is None else _need(dh, "dh", f32, (d_out,))
    dl = torch.zeros(r, dtype=torch.float32, device=dev) if dl is None else _need(dl, "dl", f32, (r,))
    dg = torch.zeros(d_in, dtype=torch.float32, device=dev) if dg is None else _need(dg, "dg", f32, (d_in,))
    dx = torch.empty((M, d_in), dtype=torch.float32, device=dev) if dx is None else _need(dx, "dx", f32, (M, d_in))
    grad_u = torch.empty((d_out, r), dtype=torch.float32, device=dev) if grad_u is None else \
        _need(grad_u, "grad_u", f32, (d_out, r))
    grad_v = torch.empty((d_in, r), dtype=torch.float32, device=dev) if grad_v is None else \
        _need(grad_v, "grad_v", f32, (d_in, r))
    if ws is None:
        ws = workspace(M, d_in, d_out, r, dev)
    _check(load().blr_backward_signs(M, d_in, d_out, r, _ptr(x), _ptr(dy), _ptr(bits_u), _ptr(bits_v), _ptr(h),
                                     _ptr(l), _ptr(g), _ptr(tape_a), _ptr(tape_c), ctypes.c_float(gscale), _ptr(dh),
                                     _ptr(dl), _ptr(dg), _ptr(dx), int(bool(accumulate_dx)), _ptr(grad_u),
                                     _ptr(grad_v), int(bool(accumulate_signs)), _ptr(ws), ws.numel(),
                                     _stream(stream)), "blr_backward_signs")
    return dh, dl, dg, dx, grad_u, grad_v


def blr_workspace_bytes_paths(M: int, d_in: int, d_out: int, r: int, paths: int) -> int:
    return int(load().blr_workspace_bytes_paths(M, d_in, d_out, r, paths))


def _paths_shapes(x, bits_u, bits_v, h, l, g):
    import torch
    f32 = (torch.float32,)
    M, d_in = _need(x, "x", f32).shape
    P, d_out = _need(h, "h", f32).shape
    r = _need(l, "l", f32, (P, l.shape[1])).shape[1]
    _need(g, "g", f32, (P, d_in))
    W = (r + 31) // 32
    _need(bits_u, "bits_u", _bits_dtypes(), (P, d_out, W))
    _need(bits_v, "bits_v", _bits_dtypes(), (P, d_in, W))
    return M, d_in, d_out, r, P


def blr_forward_paths(x, bits_u, bits_v, h, l, g, *, y=None, accumulate_y=False, tape_a=None, ws=None, stream=None):
    """Forward of a layer of P paths, fused: bits_u [P][d_out][W], bits_v
    [P][d_in][W], h [P][d_out], l [P][r], g [P][d_in]. y (+)= sum_p h_p.c_p;
    the a tape is [M][P r]. Returns (y, tape_a)."""
    import torch
    f32 = (torch.float32,)
    M, d_in, d_out, r, P = _paths_shapes(x, bits_u, bits_v, h, l, g)
    dev = x.device
    y = torch.empty((M, d_out), dtype=torch.float32, device=dev) if y is None else _need(y, "y", f32, (M, d_out))
    tape_a = torch.empty((M, P * r), dtype=torch.float32, device=dev) if tape_a is None else \
        _need(tape_a, "tape_a", f32, (M, P * r))
    if ws is None:
        ws = workspace_paths(M, d_in, d_out, r, P, dev)
    _check(load().blr_forward_paths(M, d_in, d_out, r, P, _ptr(x), _ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l),
                                    _ptr(g), _ptr(y), int(bool(accumulate_y)), _ptr(tape_a), _ptr(ws), ws.numel(),
                                    _stream(stream)), "blr_forward_paths")
    return y, tape_a


def blr_backward_paths(x, dy, bits_u, bits_v, h, l, g, tape_a, gscale: float, *, dh=None, dl=None, dg=None, dx=None,
                       accumulate_dx=False, signs=False, grad_u=None, grad_v=None, accumulate_signs=False, ws=None,
                       stream=None):
    """Backward of a layer of P paths (blr_forward_paths' tape). dh [P][d_out],
    dl [P][r], dg [P][d_in] accumulate (zeros when not given); dx is
    overwritten unless accumulate_dx. With signs (or grad_u / grad_v given)
    also the sign gradients [P][d_out][r] and [P][d_in][r]. Returns
    (dh, dl, dg, dx, grad_u, grad_v), the last two None without signs."""
    import torch
    f32 = (torch.float32,)
    M, d_in, d_out, r, P = _paths_shapes(x, bits_u, bits_v, h, l, g)
    _need(dy, "dy", f32, (M, d_out))
    _need(tape_a, "tape_a", f32, (M, P * r))
    dev = x.device
    dh = torch.zeros((P, d_out), dtype=torch.float32, device=dev) if dh is None else _need(dh, "dh", f32, (P, d_out))
    dl = torch.zeros((P, r), dtype=torch.float32, device=dev) if dl is None else _need(dl, "dl", f32, (P, r))
    dg = torch.zeros((P, d_in), dtype=torch.float32, device=dev) if dg is None else _need(dg, "dg", f32, (P, d_in))
    dx = torch.empty((M, d_in), dtype=torch.float32, device=dev) if dx is None else _need(dx, "dx", f32, (M, d_in))
    if signs or grad_u is not None or grad_v is not None:
        grad_u = torch.empty((P, d_out, r), dtype=torch.float32, device=dev) if grad_u is None else \
            _need(grad_u, "grad_u", f32, (P, d_out, r))
        grad_v = torch.empty((P, d_in, r), dtype=torch.float32, device=dev) if grad_v is None else \
            _need(grad_v, "grad_v", f32, (P, d_in, r))
    if ws is None:
        ws = workspace_paths(M, d_in, d_out, r, P, dev)
    _check(load().blr_backward_paths(M, d_in, d_out, r, P, _ptr(x), _ptr(dy), _ptr(bits_u), _ptr(bits_v), _ptr(h),
                                     _ptr(l), _ptr(g), _ptr(tape_a), ctypes.c_float(gscale), _ptr(dh), _ptr(dl),
                                     _ptr(dg), _ptr(dx), int(bool(accumulate_dx)), _ptr(grad_u), _ptr(grad_v),
                                     int(bool(accumulate_signs)), _ptr(ws), ws.numel(), _stream(stream)),
           "blr_backward_paths")
    return dh, dl, dg, dx, grad_u, grad_v


def workspace_paths(M: int, d_in: int, d_out: int, r: int, paths: int, device=None):
    import torch
    n = blr_workspace_bytes_paths(M, d_in, d_out, r, paths)
    if n == 0:
        raise BlrError(-2, "blr_workspace_bytes_paths")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def blr_plane_linear(x, plane, scale: float = 1.0, *, y=None, stream=None):
    """y [M][n] = (f16(x * scale) . plane^T) / scale with plane an f16 [n][k]
    tensor (float16 or its int16 bit patterns). Returns y."""
    import torch
    M, k = _need(x, "x", (torch.float32,)).shape
    n = _need(plane, "plane", (torch.float16, torch.int16)).shape[0]
    _need(plane, "plane", (torch.float16, torch.int16), (n, k))
    y = torch.empty((M, n), dtype=torch.float32, device=x.device) if y is None else \
        _need(y, "y", (torch.float32,), (M, n))
    _check(load().blr_plane_linear(M, n, k, _ptr(x), _ptr(plane), _ptr(y), ctypes.c_float(scale), _stream(stream)),
           "blr_plane_linear")
    return y


def blr_sumsq(a, nparts: int = 64, stream=None) -> float:
    """Sum of squares of a float32 tensor: nparts device partials, added on
    the host in f64 (the page's `sumsq`). Synchronises the stream."""
    import torch
    _need(a, "a", (torch.float32,))
    parts = torch.empty(nparts, dtype=torch.float32, device=a.device)
    _check(load().blr_sumsq(_ptr(a), a.numel(), _ptr(parts), int(nparts), _stream(stream)), "blr_sumsq")
    return float(parts.double().sum().item())


def all_finite(*tensors, stream=None) -> bool:
    """True when every element of the float32 tensors is finite (each sum
    of squares is finite; an overflowing square also reads as not finite)."""
    import math
    return all(math.isfinite(blr_sumsq(t, stream=stream)) for t in tensors)


def next_gscale(gscale: float, finite: bool, lo: float = 1.0, hi: float = 2.0 ** 24) -> float:
    """Power-of-two gradient staging scale for the next step: double it after
    a step whose gradients were finite, halve it after one that overflowed,
    within [lo, hi]."""
    g = gscale * 2.0 if finite else gscale * 0.5
    return min(max(g, lo), hi)


def blr_profile_enable(max_launches: int):
    _check(load().blr_profile_enable(int(max_launches)), "blr_profile_enable")


def blr_profile_reset():
    _check(load().blr_profile_reset(), "blr_profile_reset")


def blr_profile_read(max_kinds: int = 16) -> dict[str, tuple[int, float]]:
    """{kernel name: (launches, total ms)} of the timed launches so far."""
    names = (ctypes.c_char_p * max_kinds)()
    counts = (ctypes.c_int64 * max_kinds)()
    tot = (ctypes.c_double * max_kinds)()
    n = load().blr_profile_read(names, counts, tot, max_kinds)
    if n < 0:
        raise BlrError(n, "blr_profile_read")
    return {names[i].decode(): (int(counts[i]), float(tot[i])) for i in range(min(n, max_kinds))}
