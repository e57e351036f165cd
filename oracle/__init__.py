"""CPU oracle for the submanifold sparse convolution hot path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  The arithmetic lives in
``spconv_oracle.c`` (plain C, fp64); this module only marshals arguments.

Definitions followed (page "mlx_backend/sparse_conv_metal.py"):
  * ``forward``: out[n,co] = bias[co] + sum_k sum_ci feats[nbr[k,n],ci] w[k,ci,co]
    (module docstring formula; wrapper docstring for the layouts; the kernel
    body for skipping nbr >= N);
  * ``dgrad``: the input gradient, the adjoint of ``forward``'s linear map:
    dfeats[m,ci] = sum over (k,n) with nbr[k,n] == m of sum_co dout[n,co] w[k,ci,co]
    (from the module docstring formula; the page shows only the forward);
  * ``cast`` / ``forward_mixed``: the wrapper casts feats to w's dtype first
    (float32 -> bfloat16 to nearest, ties to even; bfloat16 -> float32 exact);
  * ``wgrad``: the weight gradient, dw[k,ci,co] = sum over n with nbr[k,n]
    present of feats[nbr[k,n],ci] dout[n,co] (the formula's derivative in w);
  * ``nmap``: nbr[k,n] = m iff coords[m] == coords[n] + dilation*o_k, else N,
    the map being an input of the page's operator whose construction the page
    does not show (offset order: x slowest, z fastest; centre k = (K-1)/2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spconv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libspconv_oracle.so")
_ASAN_PATH = os.path.join(_HERE, "_build", "libspconv_oracle_asan.so")
_lib = None

ERRORS = {0: "ok", -1: "invalid argument", -3: "coordinate out of range",
          -4: "duplicate coordinate", -7: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {code}: {ERRORS.get(code, '?')}")
        self.code = code


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with the host C compiler (no fast-math).  sanitize:
    a separate AddressSanitizer + UndefinedBehaviorSanitizer build (for a
    process that preloads the compiler's libasan), loaded when the
    SPCONV_ORACLE_LIB environment variable names it."""
    path = _ASAN_PATH if sanitize else _LIB_PATH
    if not force and os.path.exists(path):
        return path
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tmp = path + ".tmp"
    extra = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"])
    subprocess.check_call(["gcc", *extra, "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("SPCONV_ORACLE_LIB") or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.oracle_nmap.argtypes = [i32p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, i32p]
        lib.oracle_nmap_rows.argtypes = [i32p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                         i64p, ctypes.c_int64, i32p]
        lib.oracle_forward.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       i32p, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       f64p, f64p]
        lib.oracle_dgrad.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                     i32p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                     i64p, ctypes.c_int64, f64p, f64p]
        lib.oracle_wgrad.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, f64p, f64p]
        lib.oracle_morton.argtypes = [i32p, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)]
        lib.oracle_cast.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64]
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        for f in (lib.oracle_threads, lib.oracle_set_threads, lib.oracle_nmap, lib.oracle_nmap_rows, lib.oracle_forward, lib.oracle_dgrad,
                  lib.oracle_wgrad, lib.oracle_morton, lib.oracle_cast):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _check(rc):
    if rc != 0:
        raise OracleError(rc)


def _coords(coords) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(coords), dtype=np.int32)
    if c.ndim != 2 or c.shape[1] != 3:
        raise ValueError("coords must be (N,3)")
    return c


def nmap(coords, K: int = 27, dilation: int = 1) -> np.ndarray:
    """(K, N) int32 neighbour map, sentinel N."""
    c = _coords(coords)
    N = c.shape[0]
    out = np.empty((K, N), dtype=np.int32)
    _check(_load().oracle_nmap(_ptr(c, ctypes.c_int32), N, K, dilation, _ptr(out, ctypes.c_int32)))
    return out


def nmap_rows(coords, rows, K: int = 27, dilation: int = 1) -> np.ndarray:
    """(K, len(rows)) int32: the map's columns for the given voxels."""
    c = _coords(coords)
    r = np.ascontiguousarray(np.asarray(rows), dtype=np.int64)
    out = np.empty((K, r.shape[0]), dtype=np.int32)
    _check(_load().oracle_nmap_rows(_ptr(c, ctypes.c_int32), c.shape[0], K, dilation,
                                    _ptr(r, ctypes.c_int64), r.shape[0], _ptr(out, ctypes.c_int32)))
    return out


def _raw(t):
    """(contiguous numpy array, dtype code) for float32 / bfloat16 tensors or arrays."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy(), 1
            if t.dtype == torch.float32:
                return t.numpy(), 0
            raise TypeError(f"unsupported dtype {t.dtype}")
    except ImportError:
        pass
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32:
        return a, 0
    raise TypeError(f"unsupported dtype {a.dtype}")


def forward(feats, nbr, w, bias=None, with_abs: bool = True):
    """fp64 (nrows, Co) output and sum|f*w| for each column of ``nbr``.

    feats: (N, Ci) float32/bfloat16; nbr: (K, nrows) int32 with sentinel N
    (any value outside [0, N) is missing); w: (K, Ci, Co) same dtype as feats;
    bias: (Co,) float32 or None."""
    f, fd = _raw(feats)
    wa, wd = _raw(w)
    if fd != wd:
        raise TypeError("feats and w must share a dtype")
    N, Ci = f.shape
    K, Ci2, Co = wa.shape
    nb = np.ascontiguousarray(nbr, dtype=np.int32)
    if Ci2 != Ci or nb.ndim != 2 or nb.shape[0] != K:
        raise ValueError("shape mismatch")
    nrows = nb.shape[1]
    out = np.empty((nrows, Co), dtype=np.float64)
    sab = np.empty((nrows, Co), dtype=np.float64) if with_abs else None
    b = None
    if bias is not None:
        b, bd = _raw(bias)
        if bd != 0 or b.shape != (Co,):
            raise ValueError("bias must be float32 (Co,)")
    _check(_load().oracle_forward(
        f.ctypes.data, fd, N, Ci, _ptr(nb, ctypes.c_int32), K, nrows,
        wa.ctypes.data, Co, None if b is None else b.ctypes.data,
        _ptr(out, ctypes.c_double), None if sab is None else _ptr(sab, ctypes.c_double)))
    return (out, sab) if with_abs else out


def cast(x, dtype):
    """x (float32 or bfloat16 tensor) converted element-wise to ``dtype``
    (torch.float32 or torch.bfloat16) by the oracle's own rounding."""
    import torch
    a, ad = _raw(x)
    dd = {torch.float32: 0, torch.bfloat16: 1}[dtype]
    out = np.empty(a.shape, dtype=np.float32 if dd == 0 else np.int16)
    _check(_load().oracle_cast(a.ctypes.data, ad, out.ctypes.data, dd, a.size))
    t = torch.from_numpy(out)
    return t if dd == 0 else t.view(torch.bfloat16)


def forward_mixed(feats, nbr, w, bias=None, with_abs: bool = True):
    """``forward`` with feats of either dtype: feats are first cast to w's."""
    import torch
    wt = w if isinstance(w, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(w))
    return forward(cast(feats, wt.dtype), nbr, wt, bias, with_abs)


def dgrad(dout, nbr, w, rows=None, with_abs: bool = True):
    """fp64 (nrows, Ci) input gradient and sum|dout*w| for the given input rows
    (all rows when None).

    dout: (N, Co) float32/bfloat16; nbr: (K, N) int32, the forward's full map
    (sentinel N); w: (K, Ci, Co) same dtype as dout."""
    d, dd = _raw(dout)
    wa, wd = _raw(w)
    if dd != wd:
        raise TypeError("dout and w must share a dtype")
    N, Co = d.shape
    K, Ci, Co2 = wa.shape
    nb = np.ascontiguousarray(nbr, dtype=np.int32)
    if Co2 != Co or nb.shape != (K, N):
        raise ValueError("shape mismatch")
    r = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((r.shape[0], Ci), dtype=np.float64)
    sab = np.empty((r.shape[0], Ci), dtype=np.float64) if with_abs else None
    _check(_load().oracle_dgrad(d.ctypes.data, dd, N, Co, _ptr(nb, ctypes.c_int32), K, wa.ctypes.data, Ci,
                                _ptr(r, ctypes.c_int64), r.shape[0], _ptr(out, ctypes.c_double),
                                None if sab is None else _ptr(sab, ctypes.c_double)))
    return (out, sab) if with_abs else out


def wgrad(feats, dout, nbr, with_abs: bool = True):
    """fp64 (K, Ci, Co) weight gradient and sum|f*dout|.

    feats: (N, Ci), dout: (N, Co), both float32 or both bfloat16; nbr: (K, N)
    int32, the forward's map (sentinel N)."""
    f, fd = _raw(feats)
    d, dd = _raw(dout)
    if fd != dd:
        raise TypeError("feats and dout must share a dtype")
    N, Ci = f.shape
    N2, Co = d.shape
    nb = np.ascontiguousarray(nbr, dtype=np.int32)
    if N2 != N or nb.ndim != 2 or nb.shape[1] != N:
        raise ValueError("shape mismatch")
    K = nb.shape[0]
    out = np.empty((K, Ci, Co), dtype=np.float64)
    sab = np.empty((K, Ci, Co), dtype=np.float64) if with_abs else None
    _check(_load().oracle_wgrad(f.ctypes.data, d.ctypes.data, fd, N, Ci, Co, _ptr(nb, ctypes.c_int32), K,
                                _ptr(out, ctypes.c_double), None if sab is None else _ptr(sab, ctypes.c_double)))
    return (out, sab) if with_abs else out


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's later calls (OpenMP's default: all host cores)."""
    _check(_load().oracle_set_threads(int(n)))


def morton(coords) -> np.ndarray:
    """uint64 Morton codes (x,y,z biased by 2^20; z in the lowest bit)."""
    c = _coords(coords)
    out = np.empty(c.shape[0], dtype=np.uint64)
    _check(_load().oracle_morton(_ptr(c, ctypes.c_int32), c.shape[0],
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))))
    return out
