"""Thin ctypes binding of the C ABI in include/keops_mi355x.h.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of ``libkeops_mi355x.so``.  Tensors must be CUDA (HIP) float32 tensors
on one device; outputs may be passed in (``out=``, the caller-allocated
output of the "Transparent interface for billion-scale matrices" issue) or are
allocated here with ``torch.empty``.  Calls are enqueued on the current torch
stream of the tensors' device unless ``stream`` is given.  ctypes releases the
Python lock for the duration of each call.

If the library has not been built the first call raises: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkeops_mi355x.so")

KEOPS_OK = 0
KEOPS_ERR_INVALID_ARG = -1
KEOPS_ERR_UNSUPPORTED = -2
KEOPS_ERR_ALLOC = -3
KEOPS_ERR_HIP = -4
KEOPS_ERR_SCRATCH = -5
KEOPS_OPT_SPLIT_J = 1
KEOPS_OPT_FORM = 2
KEOPS_OPT_ROWS = 3
KEOPS_OPT_PROFILE = 4
KEOPS_OPT_WG_TARGET = 5
KEOPS_OPT_MFMA = 6
KEOPS_OPT_WS_CACHE = 7
KEOPS_OPT_FAIL_ALLOC = 8

_lock = threading.Lock()
_lib = None


class KeopsError(RuntimeError):
    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name}: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build the gfx950 library first "
                    "(python -m geometric_map_reduce_amd.build); there is no CPU fallback")
            L = ctypes.CDLL(LIB_PATH)
            P, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
            L.keops_gauss_sum.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_sum_noalloc.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_lse.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_grad_x.argtypes = [P, P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_grad_y.argtypes = [P, P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_grad_b.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_cg.argtypes = [P, P, i64, i32, i32, f32, f32, f32, i32, P,
                                         ctypes.POINTER(i32), ctypes.POINTER(f32), P]
            L.keops_gauss_sum_ranges.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, i64, P, P, i64, P, P]
            L.keops_gauss_lse_ranges.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, i64, P, P, i64, P, P]
            L.keops_gauss_grad_x_ranges.argtypes = [P, P, P, P, i64, i64, i32, i32, f32, P, i64, P, P, i64, P, P]
            L.keops_laplace_sum.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P]
            L.keops_gauss_max.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P, P]
            L.keops_gauss_min.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P, P]
            L.keops_kmin.argtypes = [P, P, P, i64, i64, i32, i32, f32, P, P, P]
            L.keops_set_option.argtypes = [ctypes.c_int, i64]
            L.keops_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
            L.keops_status_string.argtypes = [ctypes.c_int]
            L.keops_status_string.restype = ctypes.c_char_p
            for f in ("keops_gauss_sum", "keops_gauss_sum_noalloc", "keops_gauss_lse", "keops_gauss_grad_x",
                      "keops_gauss_grad_y", "keops_gauss_grad_b", "keops_gauss_cg", "keops_gauss_sum_ranges", "keops_gauss_lse_ranges",
                      "keops_gauss_grad_x_ranges", "keops_gauss_max", "keops_gauss_min", "keops_laplace_sum",
                      "keops_kmin",
                      "keops_set_option", "keops_version", "keops_profile_read"):
                getattr(L, f).restype = ctypes.c_int
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().keops_status_string(int(status)).decode()


def _check(name, rc):
    if rc != KEOPS_OK:
        raise KeopsError(name, rc, status_string(rc))


def _mat(t, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() == 1:
        t = t.view(-1, 1)
    if t.dim() != 2 or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D float32 CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


class _on_device:
    """Makes ``dev`` the current device for the call, switching only when it is not
    already (torch.cuda.device always switches and back, a few microseconds per call)."""
    __slots__ = ("idx", "prev")

    def __init__(self, dev):
        self.idx = dev.index
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if self.idx is not None and cur != self.idx:
            self.prev = cur
            torch.cuda.set_device(self.idx)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _out(out, shape, device, dtype=torch.float32, name="out"):
    if out is None:
        return torch.empty(shape, device=device, dtype=dtype)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or out.device != device or not out.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")
    return out


def _gauss(fn_name, x, y, b, sigma, out, stream, g=None):
    x = _mat(x, "x")
    dev = x.device
    y, b = _mat(y, "y", dev), _mat(b, "b", dev)
    M, D = x.shape
    N, E = b.shape
    if y.shape != (N, D):
        raise ValueError(f"y must be [N, D] = [{N}, {D}], got {tuple(y.shape)}")
    args = [_ptr(x), _ptr(y), _ptr(b)]
    if g is not None:
        g = _mat(g, "g", dev)
        if g.shape != (M, E):
            raise ValueError(f"g must be [M, E] = [{M}, {E}]")
        args.append(_ptr(g))
    out = _out(out, (M, D if g is not None else E), dev)
    with _on_device(dev):
        rc = getattr(lib(), fn_name)(*args, M, N, D, E, float(sigma), _ptr(out), _stream(stream, dev))
    _check(fn_name, rc)
    return out


def keops_gauss_sum(x, y, b, sigma, out=None, stream=None):
    """out[i, e] = sum_j exp(-|x_i - y_j|^2 / sigma^2) b[j, e]   (x [M,D], y [N,D], b [N,E])."""
    return _gauss("keops_gauss_sum", x, y, b, sigma, out, stream)


def keops_gauss_sum_noalloc(x, y, b, sigma, out=None, stream=None):
    """keops_gauss_sum with its workspace in the library's fixed device scratch (no device
    allocation inside the call; pass ``out`` to allocate nothing at all here either)."""
    return _gauss("keops_gauss_sum_noalloc", x, y, b, sigma, out, stream)


def keops_gauss_lse(x, y, b, sigma, out=None, stream=None):
    """out[i, e] = log sum_j exp(-|x_i - y_j|^2 / sigma^2 + b[j, e])."""
    return _gauss("keops_gauss_lse", x, y, b, sigma, out, stream)


def keops_laplace_sum(x, y, b, sigma, out=None, stream=None):
    """out[i, e] = sum_j exp(-|x_i - y_j| / sigma) b[j, e]   (the Laplacian kernel)."""
    return _gauss("keops_laplace_sum", x, y, b, sigma, out, stream)


def keops_gauss_grad_x(x, y, b, g, sigma, out=None, stream=None):
    """out[i, d] = sum_j (-2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd), the VJP of the sum with cotangent g."""
    return _gauss("keops_gauss_grad_x", x, y, b, sigma, out, stream, g=g)


def keops_gauss_grad_y(x, y, b, g, sigma, out=None, stream=None):
    """out[j, d] = sum_i (2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd): dL/dy for the cotangent g = dL/da."""
    x = _mat(x, "x")
    dev = x.device
    y, b, g = _mat(y, "y", dev), _mat(b, "b", dev), _mat(g, "g", dev)
    M, D = x.shape
    N, E = b.shape
    if y.shape != (N, D) or g.shape != (M, E):
        raise ValueError(f"need y [N, D] = [{N}, {D}] and g [M, E] = [{M}, {E}]")
    out = _out(out, (N, D), dev)
    with _on_device(dev):
        rc = lib().keops_gauss_grad_y(_ptr(x), _ptr(y), _ptr(b), _ptr(g), M, N, D, E, float(sigma), _ptr(out),
                                      _stream(stream, dev))
    _check("keops_gauss_grad_y", rc)
    return out


def keops_gauss_grad_b(x, y, g, sigma, out=None, stream=None):
    """out[j, e] = sum_i K_ij g[i, e]: dL/db for the cotangent g = dL/da."""
    x = _mat(x, "x")
    dev = x.device
    y, g = _mat(y, "y", dev), _mat(g, "g", dev)
    M, D = x.shape
    N = y.shape[0]
    E = g.shape[1]
    if y.shape != (N, D) or g.shape[0] != M:
        raise ValueError(f"need y [N, {D}] and g [M, E] with M = {M}")
    out = _out(out, (N, E), dev)
    with _on_device(dev):
        rc = lib().keops_gauss_grad_b(_ptr(x), _ptr(y), _ptr(g), M, N, D, E, float(sigma), _ptr(out),
                                      _stream(stream, dev))
    _check("keops_gauss_grad_b", rc)
    return out


def keops_gauss_cg(x, b, sigma, lam, rtol=1e-5, max_iter=1000, out=None, stream=None):
    """Solve (K + lam I) a = b, K_ij = exp(-|x_i - x_j|^2 / sigma^2), by conjugate gradients.

    Returns (a [N, E], iterations, relative true residual per column as a numpy array).
    Synchronises the stream (the residual norms are read on the host every iteration)."""
    import numpy as np
    x = _mat(x, "x")
    dev = x.device
    b = _mat(b, "b", dev)
    N, D = x.shape
    E = b.shape[1]
    if b.shape[0] != N:
        raise ValueError(f"b must have N = {N} rows")
    out = _out(out, (N, E), dev)
    it = ctypes.c_int32(0)
    res = (ctypes.c_float * max(E, 1))()
    with _on_device(dev):
        rc = lib().keops_gauss_cg(_ptr(x), _ptr(b), N, D, E, float(sigma), float(lam), float(rtol), int(max_iter),
                                  _ptr(out), ctypes.byref(it), res, _stream(stream, dev))
    _check("keops_gauss_cg", rc)
    return out, int(it.value), np.array(res[:E], np.float32)


def _host_ranges(ranges_i, slices_i, redranges_j):
    """The three range arrays as contiguous host int64 arrays (numpy or CPU tensors accepted)."""
    import numpy as np

    def arr(a, shape):
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(a, dtype=np.int64).reshape(shape))
    ri, si, rj = arr(ranges_i, (-1, 2)), arr(slices_i, (-1,)), arr(redranges_j, (-1, 2))
    if si.shape[0] != ri.shape[0]:
        raise ValueError("slices_i needs one entry per row range")
    return ri, si, rj


def _gauss_ranges(fn_name, x, y, b, sigma, ranges, out, stream, g=None):
    x = _mat(x, "x")
    dev = x.device
    y, b = _mat(y, "y", dev), _mat(b, "b", dev)
    M, D = x.shape
    N, E = b.shape
    if y.shape != (N, D):
        raise ValueError(f"y must be [N, D] = [{N}, {D}], got {tuple(y.shape)}")
    ri, si, rj = _host_ranges(*ranges)
    args = [_ptr(x), _ptr(y), _ptr(b)]
    if g is not None:
        g = _mat(g, "g", dev)
        if g.shape != (M, E):
            raise ValueError(f"g must be [M, E] = [{M}, {E}]")
        args.append(_ptr(g))
    out = _out(out, (M, D if g is not None else E), dev)
    hp = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a.size else None  # noqa: E731
    with _on_device(dev):
        rc = getattr(lib(), fn_name)(*args, M, N, D, E, float(sigma), hp(ri), ri.shape[0], hp(si), hp(rj),
                                     rj.shape[0], _ptr(out), _stream(stream, dev))
    _check(fn_name, rc)
    return out


def keops_gauss_sum_ranges(x, y, b, sigma, ranges_i, slices_i, redranges_j, out=None, stream=None):
    """Block-sparse keops_gauss_sum: row range c of ``ranges_i`` meets the j ranges
    ``redranges_j[slices_i[c-1]:slices_i[c]]``; the ranges are host arrays."""
    return _gauss_ranges("keops_gauss_sum_ranges", x, y, b, sigma, (ranges_i, slices_i, redranges_j), out, stream)


def keops_gauss_lse_ranges(x, y, b, sigma, ranges_i, slices_i, redranges_j, out=None, stream=None):
    """Block-sparse keops_gauss_lse (rows with no kept pair get -inf)."""
    return _gauss_ranges("keops_gauss_lse_ranges", x, y, b, sigma, (ranges_i, slices_i, redranges_j), out, stream)


def keops_gauss_grad_x_ranges(x, y, b, g, sigma, ranges_i, slices_i, redranges_j, out=None, stream=None):
    """Block-sparse keops_gauss_grad_x."""
    return _gauss_ranges("keops_gauss_grad_x_ranges", x, y, b, sigma, (ranges_i, slices_i, redranges_j), out,
                         stream, g=g)


def _gauss_extremum(fn_name, x, y, b, sigma, out, out_idx, stream):
    x = _mat(x, "x")
    dev = x.device
    y, b = _mat(y, "y", dev), _mat(b, "b", dev)
    M, D = x.shape
    N, E = b.shape
    if y.shape != (N, D):
        raise ValueError(f"y must be [N, D] = [{N}, {D}], got {tuple(y.shape)}")
    out = _out(out, (M, E), dev)
    out_idx = _out(out_idx, (M, E), dev, dtype=torch.int64, name="out_idx")
    with _on_device(dev):
        rc = getattr(lib(), fn_name)(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma), _ptr(out), _ptr(out_idx),
                                     _stream(stream, dev))
    _check(fn_name, rc)
    return out, out_idx


def keops_gauss_max(x, y, b, sigma, out=None, out_idx=None, stream=None):
    """(max_j K_ij b[j, e], its j) per row and column (ties: smaller j)."""
    return _gauss_extremum("keops_gauss_max", x, y, b, sigma, out, out_idx, stream)


def keops_gauss_min(x, y, b, sigma, out=None, out_idx=None, stream=None):
    """(min_j K_ij b[j, e], its j) per row and column (ties: smaller j)."""
    return _gauss_extremum("keops_gauss_min", x, y, b, sigma, out, out_idx, stream)


def keops_kmin(x, y, K, out_d=None, out_idx=None, stream=None):
    """K smallest |x_i - y_j|^2 per row (ascending, ties by smaller j) and their int64 indices."""
    x = _mat(x, "x")
    dev = x.device
    y = _mat(y, "y", dev)
    M, D = x.shape
    N = y.shape[0]
    if y.shape[1] != D:
        raise ValueError("x and y must have the same number of columns")
    out_d = _out(out_d, (M, K), dev, name="out_d")
    out_idx = _out(out_idx, (M, K), dev, dtype=torch.int64, name="out_idx")
    with _on_device(dev):
        # b and sigma of the uniform argument list are not read by K-min
        rc = lib().keops_kmin(_ptr(x), _ptr(y), None, M, N, D, int(K), 1.0, _ptr(out_d), _ptr(out_idx),
                              _stream(stream, dev))
    _check("keops_kmin", rc)
    return out_d, out_idx


def keops_set_option(option: int, value: int) -> None:
    """Process-wide scheduling switch (KEOPS_OPT_*); 0 restores the automatic choice."""
    _check("keops_set_option", lib().keops_set_option(int(option), int(value)))


def keops_profile_read() -> tuple[float, int]:
    """(summed pass-1 kernel milliseconds, launches) recorded while KEOPS_OPT_PROFILE was 1."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check("keops_profile_read", lib().keops_profile_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def keops_version() -> int:
    return int(lib().keops_version())
