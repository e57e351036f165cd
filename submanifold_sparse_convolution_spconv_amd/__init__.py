"""Submanifold sparse 3D convolution on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libspconv_mi355x.so`` (declared in
``include/spconv_mi355x.h``).  Every step of the computation runs in the HIP
library; this module only checks tensor metadata, allocates the caller-owned
device buffers with PyTorch and passes pointers and the current HIP stream.
There is no fallback: if the library cannot be loaded, calls raise.

Operation (page "mlx_backend/sparse_conv_metal.py"):
    out[n, co] = bias[co] + sum_k sum_ci feats[nbr[k, n], ci] * w[k, ci, co]
with nbr a (K, N) int32 map whose value N marks a missing neighbour.

Functions carry the C entry points' names:
    spconv_nmap_sizes(N, K) -> (arena_bytes, workspace_bytes)
    spconv_build_nmap(coords, K=27, dilation=1) -> NMap
    spconv_nmap_wrap(nbr) -> NMap
    spconv_nmap_export(nmap) -> (nbr (K,N) int32, order (N,) int32)
    spconv_nmap_info(nmap) -> dict(N, K, dilation, valid_pairs)
    spconv_forward(feats, nmap, w, bias=None, out=None) -> out
    spconv_pack_weights_size(K, Ci, Co, dtype) -> bytes
    spconv_pack_weights(w) -> wpack (uint8 tensor; empty when there is no packed form)
    spconv_forward_packed(feats, nmap, w, wpack, bias=None, out=None) -> out
    spconv_forward_mixed(feats, nmap, w, bias=None, out=None) -> out  (feats cast to w's dtype)
    spconv_build_nmap_batched(coords (N,4) b,x,y,z, batches, K=27, dilation=1) -> NMap
    spconv_dgrad(dout, nmap, w) -> dfeats
    spconv_dgrad_noalloc(dout, nmap, w, out) -> out  (no workspace: a fixed scratch in the library)
    spconv_wgrad(feats, dout, nmap) -> dw
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SpconvError", "NMap", "load_library", "library_path",
    "spconv_nmap_sizes", "spconv_build_nmap", "spconv_nmap_wrap", "spconv_nmap_export",
    "spconv_nmap_info", "spconv_forward", "spconv_nmap_destroy",
    "spconv_pack_weights_size", "spconv_pack_weights", "spconv_forward_packed", "spconv_forward_mixed",
    "spconv_forward_mixed_workspace_size",
    "spconv_build_nmap_batched", "spconv_dgrad_workspace_size", "spconv_dgrad", "spconv_dgrad_noalloc",
    "SPCONV_NOALLOC_SCRATCH_BYTES",
    "spconv_wgrad_workspace_size", "spconv_wgrad",
    "SPCONV_F32", "SPCONV_BF16", "STATUS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPCONV_LIB may name another build of the library (the host-sanitized one)
_LIB_PATH = os.environ.get("SPCONV_LIB") or os.path.join(_PKG, "libspconv_mi355x.so")

SPCONV_F32 = 0
SPCONV_BF16 = 1
STATUS = {0: "SPCONV_OK", -1: "SPCONV_E_INVALID", -2: "SPCONV_E_UNSUPPORTED",
          -3: "SPCONV_E_COORD_RANGE", -4: "SPCONV_E_DUPLICATE", -5: "SPCONV_E_WORKSPACE",
          -6: "SPCONV_E_HIP"}

_lib = None


class SpconvError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the HIP library, building it first only if no build exists."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz, i64, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
    lib.spconv_abi_version.argtypes = []
    lib.spconv_abi_version.restype = i32
    lib.spconv_nmap_sizes.argtypes = [i64, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.spconv_build_nmap.argtypes = [vp, i64, i32, i32, vp, sz, vp, sz, vp, ctypes.POINTER(vp)]
    lib.spconv_build_nmap_batched.argtypes = [vp, i64, i32, i32, i32, vp, sz, vp, sz, vp, ctypes.POINTER(vp)]
    lib.spconv_nmap_wrap.argtypes = [vp, i64, i32, vp, sz, vp, ctypes.POINTER(vp)]
    lib.spconv_nmap_export.argtypes = [vp, vp, vp, vp]
    lib.spconv_nmap_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                     ctypes.POINTER(i32), ctypes.POINTER(i64), vp]
    lib.spconv_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.spconv_forward_mixed.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, sz, vp]
    lib.spconv_forward_mixed_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.POINTER(sz)]
    lib.spconv_forward_mixed_workspace_size.restype = i32
    for f in (lib.spconv_nmap_sizes, lib.spconv_build_nmap, lib.spconv_build_nmap_batched, lib.spconv_nmap_wrap,
              lib.spconv_nmap_export, lib.spconv_nmap_info, lib.spconv_forward, lib.spconv_forward_mixed):
        f.restype = i32
    lib.spconv_pack_weights_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.spconv_pack_weights_size.restype = i32
    lib.spconv_pack_weights.argtypes = [vp, i32, i32, i32, i32, vp, sz, vp]
    lib.spconv_pack_weights.restype = i32
    lib.spconv_forward_packed.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.spconv_forward_packed.restype = i32
    lib.spconv_dgrad_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.spconv_dgrad_workspace_size.restype = i32
    lib.spconv_dgrad.argtypes = [vp, vp, vp, vp, sz, vp, i32, i32, i32, vp]
    lib.spconv_dgrad.restype = i32
    lib.spconv_dgrad_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
    lib.spconv_dgrad_noalloc.restype = i32
    lib.spconv_wgrad_workspace_size.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.spconv_wgrad_workspace_size.restype = i32
    lib.spconv_wgrad.argtypes = [vp, vp, vp, vp, sz, vp, i32, i32, i32, vp]
    lib.spconv_wgrad.restype = i32
    lib.spconv_nmap_destroy.argtypes = [vp]
    lib.spconv_nmap_destroy.restype = None
    lib.spconv_status_string.argtypes = [i32]
    lib.spconv_status_string.restype = ctypes.c_char_p
    lib.spconv_last_error.argtypes = []
    lib.spconv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int, where: str):
    if rc != 0:
        raise SpconvError(rc, where, load_library().spconv_last_error().decode())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def spconv_nmap_sizes(N: int, K: int):
    a, w = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().spconv_nmap_sizes(N, K, ctypes.byref(a), ctypes.byref(w)),
           "spconv_nmap_sizes")
    return a.value, w.value


class NMap:
    """A built (or wrapped) neighbour map: the C handle plus the arena tensor
    that holds its device data."""

    def __init__(self, handle, arena, N, K, dilation, device):
        self._h = handle
        self.arena = arena
        self.N, self.K, self.dilation, self.device = N, K, dilation, device

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("neighbour map already destroyed")
        return self._h

    def destroy(self):
        if self._h is not None and _lib is not None:
            _lib.spconv_nmap_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    @property
    def valid_pairs(self) -> int:
        return spconv_nmap_info(self)["valid_pairs"]

    def export(self):
        return spconv_nmap_export(self)


def spconv_build_nmap(coords, K: int = 27, dilation: int = 1, workspace=None) -> NMap:
    """coords: int32 CUDA tensor (N, 3).  Returns an NMap (arena owned by it)."""
    import torch
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 3 or not coords.is_cuda:
        raise ValueError("coords must be an int32 CUDA tensor of shape (N, 3)")
    coords = coords.contiguous()
    N = coords.shape[0]
    lib = load_library()
    arena_b, ws_b = spconv_nmap_sizes(N, K)
    dev = coords.device
    arena = torch.empty(arena_b, dtype=torch.uint8, device=dev)
    ws = workspace
    if ws is None or ws.numel() < ws_b:
        ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    h = ctypes.c_void_p()
    with torch.cuda.device(dev):
        rc = lib.spconv_build_nmap(_ptr(coords), N, K, dilation, _ptr(arena), arena_b,
                                   _ptr(ws), ws.numel(), _stream(dev), ctypes.byref(h))
    _check(rc, "spconv_build_nmap")
    return NMap(h, arena, N, K, dilation, dev)


def spconv_build_nmap_batched(coords, batches: int, K: int = 27, dilation: int = 1, workspace=None) -> NMap:
    """coords: int32 CUDA tensor (N, 4) of (b, x, y, z), b in [0, batches);
    voxels are neighbours only within one batch.  Returns an NMap."""
    import torch
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4 or not coords.is_cuda:
        raise ValueError("coords must be an int32 CUDA tensor of shape (N, 4)")
    coords = coords.contiguous()
    N = coords.shape[0]
    lib = load_library()
    arena_b, ws_b = spconv_nmap_sizes(N, K)
    dev = coords.device
    arena = torch.empty(arena_b, dtype=torch.uint8, device=dev)
    ws = workspace
    if ws is None or ws.numel() < ws_b:
        ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    h = ctypes.c_void_p()
    with torch.cuda.device(dev):
        rc = lib.spconv_build_nmap_batched(_ptr(coords), N, batches, K, dilation, _ptr(arena), arena_b,
                                           _ptr(ws), ws.numel(), _stream(dev), ctypes.byref(h))
    _check(rc, "spconv_build_nmap_batched")
    return NMap(h, arena, N, K, dilation, dev)


def spconv_nmap_wrap(nbr) -> NMap:
    """nbr: int32 CUDA tensor (K, N), element [k, n], sentinel N."""
    import torch
    if nbr.dtype != torch.int32 or nbr.dim() != 2 or not nbr.is_cuda:
        raise ValueError("nbr must be an int32 CUDA tensor of shape (K, N)")
    nbr = nbr.contiguous()
    K, N = nbr.shape
    lib = load_library()
    arena_b, _ = spconv_nmap_sizes(N, K)
    dev = nbr.device
    arena = torch.empty(arena_b, dtype=torch.uint8, device=dev)
    h = ctypes.c_void_p()
    with torch.cuda.device(dev):
        rc = lib.spconv_nmap_wrap(_ptr(nbr), N, K, _ptr(arena), arena_b, _stream(dev), ctypes.byref(h))
    _check(rc, "spconv_nmap_wrap")
    return NMap(h, arena, N, K, 1, dev)


def spconv_nmap_export(nmap: NMap):
    """(nbr (K, N) int32, order (N,) int32) on the map's device, caller order."""
    import torch
    nbr = torch.empty((nmap.K, nmap.N), dtype=torch.int32, device=nmap.device)
    order = torch.empty((nmap.N,), dtype=torch.int32, device=nmap.device)
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_nmap_export(nmap.handle, _ptr(nbr), _ptr(order), _stream(nmap.device))
    _check(rc, "spconv_nmap_export")
    return nbr, order


def spconv_nmap_info(nmap: NMap) -> dict:
    import torch
    N, vp = ctypes.c_int64(), ctypes.c_int64()
    K, d = ctypes.c_int(), ctypes.c_int()
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_nmap_info(nmap.handle, ctypes.byref(N), ctypes.byref(K),
                                             ctypes.byref(d), ctypes.byref(vp), _stream(nmap.device))
    _check(rc, "spconv_nmap_info")
    return {"N": N.value, "K": K.value, "dilation": d.value, "valid_pairs": vp.value}


def spconv_nmap_destroy(nmap: NMap):
    nmap.destroy()


def _forward_args(feats, nmap: NMap, w, bias, out, mixed=False):
    import torch
    dt = {torch.float32: SPCONV_F32, torch.bfloat16: SPCONV_BF16}.get(w.dtype)
    if dt is None or feats.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("feats and w must be float32 or bfloat16")
    if not mixed and feats.dtype != w.dtype:
        raise ValueError("feats and w must both be float32 or both bfloat16")
    if w.dim() != 3 or w.shape[0] != nmap.K or feats.dim() != 2 or feats.shape[1] != w.shape[1]:
        raise ValueError("expected feats (N, Ci) and w (K, Ci, Co) matching the map")
    if feats.shape[0] not in (nmap.N, nmap.N + 1):
        raise ValueError("feats must have N or N+1 rows")
    for t in (feats, w):
        if not t.is_cuda or t.device != nmap.device:
            raise ValueError("tensors must live on the map's device")
    Co = w.shape[2]
    feats = feats.contiguous()
    w = w.contiguous()
    if bias is not None:
        if bias.dtype != torch.float32 or bias.shape != (Co,) or bias.device != nmap.device:
            raise ValueError("bias must be float32 (Co,) on the map's device")
        bias = bias.contiguous()
    if out is None:
        out = torch.empty((nmap.N, Co), dtype=w.dtype, device=nmap.device)
    elif out.shape != (nmap.N, Co) or out.dtype != w.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (N, Co) tensor of w's dtype")
    return feats, w, bias, out, dt


def spconv_forward(feats, nmap: NMap, w, bias=None, out=None):
    """feats (N or N+1, Ci), w (K, Ci, Co): both float32 or both bfloat16, CUDA.
    bias: float32 (Co,) or None.  Returns out (N, Co) in w's dtype."""
    import torch
    feats, w, bias, out, dt = _forward_args(feats, nmap, w, bias, out)
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_forward(_ptr(feats), nmap.handle, _ptr(w), _ptr(bias), _ptr(out),
                                           w.shape[1], w.shape[2], dt, _stream(nmap.device))
    _check(rc, "spconv_forward")
    return out


def spconv_forward_mixed_workspace_size(N: int, Ci: int, feats_dtype: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spconv_forward_mixed_workspace_size(N, Ci, feats_dtype, dtype, ctypes.byref(n)),
           "spconv_forward_mixed_workspace_size")
    return n.value


def spconv_forward_mixed(feats, nmap: NMap, w, bias=None, out=None, workspace=None, wpack=None):
    """spconv_forward with feats float32 or bfloat16 independently of w: feats
    are converted to w's dtype (fp32 -> bf16 rounds to nearest even).  With a
    uint8 device ``workspace`` of spconv_forward_mixed_workspace_size bytes,
    fp32 feats are cast by a separate pass first; without one, in the gather.
    ``wpack`` (spconv_pack_weights(w)) is optional.  Returns out (N, Co) in
    w's dtype."""
    import torch
    feats, w, bias, out, dt = _forward_args(feats, nmap, w, bias, out, mixed=True)
    fdt = SPCONV_F32 if feats.dtype == torch.float32 else SPCONV_BF16
    if wpack is not None:
        if wpack.dtype != torch.uint8 or wpack.device != nmap.device:
            raise ValueError("wpack must be the uint8 tensor from spconv_pack_weights on the map's device")
        if wpack.numel() < spconv_pack_weights_size(nmap.K, w.shape[1], w.shape[2], dt):
            raise ValueError("wpack is smaller than spconv_pack_weights_size")
    ws, wsb = None, 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != nmap.device:
            raise ValueError("workspace must be a contiguous uint8 tensor on the map's device")
        ws, wsb = workspace, workspace.numel()
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_forward_mixed(_ptr(feats), fdt, nmap.handle, _ptr(w),
                                                 _ptr(wpack) if wpack is not None and wpack.numel() else None,
                                                 _ptr(bias), _ptr(out), w.shape[1], w.shape[2], dt, _ptr(ws), wsb,
                                                 _stream(nmap.device))
    _check(rc, "spconv_forward_mixed")
    return out


def spconv_pack_weights_size(K: int, Ci: int, Co: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spconv_pack_weights_size(K, Ci, Co, dtype, ctypes.byref(n)),
           "spconv_pack_weights_size")
    return n.value


def spconv_pack_weights(w, out=None):
    """Packed copy of w (K, Ci, Co) for spconv_forward_packed: a uint8 device
    tensor, empty when the forward has no packed form for this configuration."""
    import torch
    dt = {torch.float32: SPCONV_F32, torch.bfloat16: SPCONV_BF16}.get(w.dtype)
    if dt is None or w.dim() != 3 or not w.is_cuda:
        raise ValueError("w must be a float32 or bfloat16 (K, Ci, Co) CUDA tensor")
    w = w.contiguous()
    K, Ci, Co = w.shape
    n = spconv_pack_weights_size(K, Ci, Co, dt)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    elif out.dtype != torch.uint8 or out.numel() < n or out.device != w.device:
        raise ValueError("out must be a uint8 tensor of at least spconv_pack_weights_size bytes")
    with torch.cuda.device(w.device):
        rc = load_library().spconv_pack_weights(_ptr(w), K, Ci, Co, dt, _ptr(out) if n else None, n,
                                                _stream(w.device))
    _check(rc, "spconv_pack_weights")
    return out


def spconv_forward_packed(feats, nmap: NMap, w, wpack, bias=None, out=None):
    """spconv_forward with wpack = spconv_pack_weights(w)."""
    import torch
    feats, w, bias, out, dt = _forward_args(feats, nmap, w, bias, out)
    if wpack.dtype != torch.uint8 or wpack.device != nmap.device:
        raise ValueError("wpack must be the uint8 tensor from spconv_pack_weights on the map's device")
    if wpack.numel() < spconv_pack_weights_size(nmap.K, w.shape[1], w.shape[2], dt):
        raise ValueError("wpack is smaller than spconv_pack_weights_size")
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_forward_packed(_ptr(feats), nmap.handle, _ptr(w),
                                                  _ptr(wpack) if wpack.numel() else None, _ptr(bias),
                                                  _ptr(out), w.shape[1], w.shape[2], dt, _stream(nmap.device))
    _check(rc, "spconv_forward_packed")
    return out


def spconv_dgrad_workspace_size(K: int, Ci: int, Co: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spconv_dgrad_workspace_size(K, Ci, Co, dtype, ctypes.byref(n)),
           "spconv_dgrad_workspace_size")
    return n.value


def spconv_dgrad(dout, nmap: NMap, w, out=None, workspace=None):
    """Input gradient of spconv_forward: dout (N, Co) and w (K, Ci, Co), both
    float32 or both bfloat16, CUDA; returns dfeats (N, Ci) in w's dtype.  The
    map must come from spconv_build_nmap.  workspace: a uint8 tensor of at least
    spconv_dgrad_workspace_size bytes (allocated when None)."""
    import torch
    dt = {torch.float32: SPCONV_F32, torch.bfloat16: SPCONV_BF16}.get(w.dtype)
    if dt is None or dout.dtype != w.dtype:
        raise ValueError("dout and w must both be float32 or both bfloat16")
    if w.dim() != 3 or w.shape[0] != nmap.K or dout.dim() != 2 or dout.shape != (nmap.N, w.shape[2]):
        raise ValueError("expected dout (N, Co) and w (K, Ci, Co) matching the map")
    for t in (dout, w):
        if not t.is_cuda or t.device != nmap.device:
            raise ValueError("tensors must live on the map's device")
    K, Ci, Co = w.shape
    dout = dout.contiguous()
    w = w.contiguous()
    n = spconv_dgrad_workspace_size(K, Ci, Co, dt)
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=nmap.device)
    elif workspace.dtype != torch.uint8 or workspace.numel() < n or workspace.device != nmap.device:
        raise ValueError("workspace must be a uint8 tensor of at least spconv_dgrad_workspace_size bytes")
    if out is None:
        out = torch.empty((nmap.N, Ci), dtype=w.dtype, device=nmap.device)
    elif out.shape != (nmap.N, Ci) or out.dtype != w.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (N, Ci) tensor of w's dtype")
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_dgrad(_ptr(dout), nmap.handle, _ptr(w), _ptr(workspace), workspace.numel(),
                                         _ptr(out), Ci, Co, dt, _stream(nmap.device))
    _check(rc, "spconv_dgrad")
    return out


SPCONV_NOALLOC_SCRATCH_BYTES = 16 << 20


def spconv_dgrad_noalloc(dout, nmap: NMap, w, out):
    """spconv_dgrad without a workspace: the library's fixed per-device scratch
    (SPCONV_NOALLOC_SCRATCH_BYTES) holds the mirrored weights, so the C call
    allocates nothing.  ``out`` (N, Ci) in w's dtype is required, so this
    function allocates nothing either.  Calls that overlap in time on one
    device race on the scratch."""
    import torch
    dt = {torch.float32: SPCONV_F32, torch.bfloat16: SPCONV_BF16}.get(w.dtype)
    if dt is None or dout.dtype != w.dtype:
        raise ValueError("dout and w must both be float32 or both bfloat16")
    if w.dim() != 3 or w.shape[0] != nmap.K or dout.dim() != 2 or dout.shape != (nmap.N, w.shape[2]):
        raise ValueError("expected dout (N, Co) and w (K, Ci, Co) matching the map")
    if not (dout.is_contiguous() and w.is_contiguous()):
        raise ValueError("dout and w must be contiguous (no copies are made)")
    K, Ci, Co = w.shape
    if out is None or out.shape != (nmap.N, Ci) or out.dtype != w.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (N, Ci) tensor of w's dtype")
    for t in (dout, w, out):
        if not t.is_cuda or t.device != nmap.device:
            raise ValueError("tensors must live on the map's device")
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_dgrad_noalloc(_ptr(dout), nmap.handle, _ptr(w), _ptr(out), Ci, Co, dt,
                                                 _stream(nmap.device))
    _check(rc, "spconv_dgrad_noalloc")
    return out


def spconv_wgrad_workspace_size(N: int, K: int, Ci: int, Co: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spconv_wgrad_workspace_size(N, K, Ci, Co, dtype, ctypes.byref(n)),
           "spconv_wgrad_workspace_size")
    return n.value


def spconv_wgrad(feats, dout, nmap: NMap, out=None, workspace=None):
    """Weight gradient of spconv_forward: feats (N or N+1, Ci) and dout (N, Co),
    both float32 or both bfloat16, CUDA; returns dw (K, Ci, Co) in their dtype.
    workspace: a uint8 tensor of at least spconv_wgrad_workspace_size bytes
    (allocated when None)."""
    import torch
    dt = {torch.float32: SPCONV_F32, torch.bfloat16: SPCONV_BF16}.get(feats.dtype)
    if dt is None or dout.dtype != feats.dtype:
        raise ValueError("feats and dout must both be float32 or both bfloat16")
    if feats.dim() != 2 or dout.dim() != 2 or feats.shape[0] not in (nmap.N, nmap.N + 1) or dout.shape[0] != nmap.N:
        raise ValueError("expected feats (N or N+1, Ci) and dout (N, Co) matching the map")
    for t in (feats, dout):
        if not t.is_cuda or t.device != nmap.device:
            raise ValueError("tensors must live on the map's device")
    Ci, Co = feats.shape[1], dout.shape[1]
    feats = feats.contiguous()
    dout = dout.contiguous()
    n = spconv_wgrad_workspace_size(nmap.N, nmap.K, Ci, Co, dt)
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=nmap.device)
    elif workspace.dtype != torch.uint8 or workspace.numel() < n or workspace.device != nmap.device:
        raise ValueError("workspace must be a uint8 tensor of at least spconv_wgrad_workspace_size bytes")
    if out is None:
        out = torch.empty((nmap.K, Ci, Co), dtype=feats.dtype, device=nmap.device)
    elif out.shape != (nmap.K, Ci, Co) or out.dtype != feats.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (K, Ci, Co) tensor of feats' dtype")
    with torch.cuda.device(nmap.device):
        rc = load_library().spconv_wgrad(_ptr(feats), _ptr(dout), nmap.handle, _ptr(workspace), workspace.numel(),
                                         _ptr(out), Ci, Co, dt, _stream(nmap.device))
    _check(rc, "spconv_wgrad")
    return out
