"""Seeded synthetic inputs for the submanifold sparse convolution hot path.

This module only draws inputs: voxel coordinates (the active-site set and its
caller order) and the feature / weight / bias values.  It holds none of the
convolution's arithmetic, so both the CPU oracle and the GPU library can be fed
from it without sharing any code with each other.

Five workloads are defined, named by their geometry and sizes:

  uniform32   4,096 voxels drawn uniformly without replacement from a 32^3
              grid, K=27, Ci=Co=32, fp32.
  shell64     the spherical shell | |v-(32,32,32)| - 28 | < 1.5 in a 64^3 grid,
              K=27, Ci=Co=64, bf16 in / bf16 out.
  surf256     16 random sphere shells + 8 random planes in a 256^3 grid
              (about 1.0M surface voxels), K=27, Ci=Co=128, bf16.
  surf1024    10 shells + 5 planes in a 1024^3 grid (about 11M voxels),
              K=27, Ci=128, Co=64, bf16.
  surf512d2   10 shells + 5 planes in a 512^3 grid (about 2.2M voxels),
              K=27 at dilation 2, Ci=32, Co=256, fp32.

Recipe (all numpy PCG64 ``default_rng``):
  * geometry seed i (workload index 1..5), caller-order shuffle seed 1000+i,
    value seed 100+i with draws in the order feats, w, bias;
  * "N(0, v)" means variance v: feats ~ N(0,1), w ~ N(0, 1/(27*Ci)),
    bias ~ N(0, 0.1); values are drawn as float32 normals and, for bf16
    workloads, rounded to bfloat16 with round-to-nearest-even (bias stays fp32);
  * sphere shell j: centre ~ U[0,G)^3 then radius ~ U[Rmin,Rmax]; all shells are
    drawn before the planes; plane j: unit normal from a standard normal 3-vector,
    then a point ~ U[G/4, 3G/4)^3;
  * voxel v of [0,G)^3 is active iff some shell has | |v-c| - R | < 0.5 or some
    plane has |n.(v-p)| < 0.5, evaluated in float64.

The surface workloads enumerate candidate voxels per surface instead of
evaluating every voxel of the dense grid (1024^3 would not fit comfortably in
memory); each candidate is then tested with exactly the float64 expression a
dense evaluation would use, and the candidate ranges carry a one-voxel margin,
so the active set is the same as the dense one (``dense_surface_mask`` is kept
for tests that check this on small grids).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "by_name", "geometry", "values", "make",
    "surface_coords", "dense_surface_mask", "uniform_coords", "shell_coords",
    "raster_coords", "linear_to_xyz",
]


@dataclass(frozen=True)
class Workload:
    index: int            # 1..5
    name: str
    kind: str             # "uniform" | "shell" | "surfaces"
    grid: int             # G
    K: int
    dilation: int
    Ci: int
    Co: int
    dtype: str            # "f32" | "bf16"
    params: dict = field(default_factory=dict)

    @property
    def geom_seed(self) -> int:
        return self.index

    @property
    def shuffle_seed(self) -> int:
        return 1000 + self.index

    @property
    def value_seed(self) -> int:
        return 100 + self.index


WORKLOADS = [
    Workload(1, "uniform32", "uniform", 32, 27, 1, 32, 32, "f32", {"n": 4096}),
    Workload(2, "shell64", "shell", 64, 27, 1, 64, 64, "bf16",
             {"center": (32.0, 32.0, 32.0), "radius": 28.0, "half_width": 1.5}),
    Workload(3, "surf256", "surfaces", 256, 27, 1, 128, 128, "bf16",
             {"n_shells": 16, "r_min": 16.0, "r_max": 96.0, "n_planes": 8}),
    Workload(4, "surf1024", "surfaces", 1024, 27, 1, 128, 64, "bf16",
             {"n_shells": 10, "r_min": 64.0, "r_max": 384.0, "n_planes": 5}),
    Workload(5, "surf512d2", "surfaces", 512, 27, 2, 32, 256, "f32",
             {"n_shells": 10, "r_min": 32.0, "r_max": 192.0, "n_planes": 5}),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name or str(w.index) == str(name):
            return w
    raise KeyError(name)


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------

def linear_to_xyz(lin: np.ndarray, G: int) -> np.ndarray:
    """Raster index (x slowest, z fastest) -> int32 (n,3) coordinates."""
    lin = np.asarray(lin, dtype=np.int64)
    return np.stack([lin // (G * G), (lin // G) % G, lin % G], axis=1).astype(np.int32)


def uniform_coords(G: int, n: int, seed: int) -> np.ndarray:
    """n distinct voxels of [0,G)^3, uniform without replacement; draw order kept."""
    rng = np.random.default_rng(seed)
    lin = rng.choice(G ** 3, size=n, replace=False)
    return linear_to_xyz(lin, G)


def shell_coords(G: int, center, radius: float, half_width: float) -> np.ndarray:
    """Voxels with | |v-c| - R | < half_width, raster order (deterministic)."""
    ax = np.arange(G, dtype=np.float64)
    x, y, z = np.meshgrid(ax, ax, ax, indexing="ij")
    d = np.sqrt((x - center[0]) * (x - center[0]) + (y - center[1]) * (y - center[1])
                + (z - center[2]) * (z - center[2]))
    mask = np.abs(d - radius) < half_width
    return linear_to_xyz(np.flatnonzero(mask.ravel()), G)


def _draw_surfaces(G: int, n_shells: int, r_min: float, r_max: float,
                   n_planes: int, seed: int):
    rng = np.random.default_rng(seed)
    shells = []
    for _ in range(n_shells):
        c = rng.uniform(0.0, G, size=3)
        r = float(rng.uniform(r_min, r_max))
        shells.append((c, r))
    planes = []
    for _ in range(n_planes):
        nrm = rng.standard_normal(3)
        nrm = nrm / np.sqrt(np.sum(nrm * nrm))
        p = rng.uniform(G / 4.0, 3.0 * G / 4.0, size=3)
        planes.append((nrm, p))
    return shells, planes


def _shell_pred(x, y, z, c, r):
    dx = x - c[0]
    dy = y - c[1]
    dz = z - c[2]
    return np.abs(np.sqrt(dx * dx + dy * dy + dz * dz) - r) < 0.5


def _plane_pred(x, y, z, nrm, p):
    return np.abs(nrm[0] * (x - p[0]) + nrm[1] * (y - p[1]) + nrm[2] * (z - p[2])) < 0.5


def dense_surface_mask(G: int, shells, planes) -> np.ndarray:
    """Dense float64 evaluation over all of [0,G)^3 (small G only)."""
    ax = np.arange(G, dtype=np.float64)
    x, y, z = np.meshgrid(ax, ax, ax, indexing="ij")
    m = np.zeros((G, G, G), dtype=bool)
    for c, r in shells:
        m |= _shell_pred(x, y, z, c, r)
    for nrm, p in planes:
        m |= _plane_pred(x, y, z, nrm, p)
    return m


def _mark_shell(occ: np.ndarray, G: int, c, r: float) -> None:
    lo = max(0, int(math.floor(c[0] - r - 0.5)) - 1)
    hi = min(G - 1, int(math.ceil(c[0] + r + 0.5)) + 1)
    ylo = max(0, int(math.floor(c[1] - r - 0.5)) - 1)
    yhi = min(G - 1, int(math.ceil(c[1] + r + 0.5)) + 1)
    if lo > hi or ylo > yhi:
        return
    xs = np.arange(lo, hi + 1, dtype=np.float64)
    ys = np.arange(ylo, yhi + 1, dtype=np.float64)
    X, Y = np.meshgrid(xs, ys, indexing="ij")
    X = X.ravel()
    Y = Y.ravel()
    rho2 = (X - c[0]) ** 2 + (Y - c[1]) ** 2
    outer2 = (r + 0.5) ** 2 - rho2
    keep = outer2 > -4.0 * (r + 2.0)          # generous: margin handled below
    X, Y, rho2, outer2 = X[keep], Y[keep], rho2[keep], outer2[keep]
    zmax = np.sqrt(np.maximum(outer2, 0.0))
    zmin = np.sqrt(np.maximum((r - 0.5) ** 2 - rho2, 0.0))
    # two candidate intervals of z per (x,y): c_z +- [zmin, zmax], one-voxel margin
    segs = []
    for sign in (-1.0, 1.0):
        a = c[2] + sign * zmax
        b = c[2] + sign * zmin
        zl = np.floor(np.minimum(a, b)) - 1.0
        zh = np.ceil(np.maximum(a, b)) + 1.0
        zl = np.clip(zl, 0, G - 1)
        zh = np.clip(zh, 0, G - 1)
        segs.append((zl, zh))
    for zl, zh in segs:
        cnt = (zh - zl + 1).astype(np.int64)
        cnt[cnt < 0] = 0
        tot = int(cnt.sum())
        if tot == 0:
            continue
        rep = np.repeat(np.arange(len(cnt)), cnt)
        start = np.repeat(np.cumsum(cnt) - cnt, cnt)
        Z = zl[rep] + (np.arange(tot) - start)
        Xc = X[rep]
        Yc = Y[rep]
        ok = _shell_pred(Xc, Yc, Z, c, r)
        lin = (Xc[ok].astype(np.int64) * G + Yc[ok].astype(np.int64)) * G + Z[ok].astype(np.int64)
        occ[lin] = True


def _mark_plane(occ: np.ndarray, G: int, nrm, p) -> None:
    a = int(np.argmax(np.abs(nrm)))           # solve for the dominant axis
    o1, o2 = [ax for ax in range(3) if ax != a]
    g = np.arange(G, dtype=np.float64)
    U, V = np.meshgrid(g, g, indexing="ij")
    U = U.ravel()
    V = V.ravel()
    s = nrm[o1] * (U - p[o1]) + nrm[o2] * (V - p[o2])
    # n_a (v_a - p_a) in (-0.5 - s, 0.5 - s)
    t1 = p[a] + (-0.5 - s) / nrm[a]
    t2 = p[a] + (0.5 - s) / nrm[a]
    vl = np.clip(np.floor(np.minimum(t1, t2)) - 1.0, 0, G - 1)
    vh = np.clip(np.ceil(np.maximum(t1, t2)) + 1.0, 0, G - 1)
    cnt = (vh - vl + 1).astype(np.int64)
    inb = (np.maximum(t1, t2) >= -2.0) & (np.minimum(t1, t2) <= G + 1.0)
    cnt[~inb] = 0
    tot = int(cnt.sum())
    if tot == 0:
        return
    rep = np.repeat(np.arange(len(cnt)), cnt)
    start = np.repeat(np.cumsum(cnt) - cnt, cnt)
    W = vl[rep] + (np.arange(tot) - start)
    coords = [None, None, None]
    coords[a] = W
    coords[o1] = U[rep]
    coords[o2] = V[rep]
    ok = _plane_pred(coords[0], coords[1], coords[2], nrm, p)
    lin = (coords[0][ok].astype(np.int64) * G + coords[1][ok].astype(np.int64)) * G \
        + coords[2][ok].astype(np.int64)
    occ[lin] = True


def surface_coords(G: int, n_shells: int, r_min: float, r_max: float,
                   n_planes: int, seed: int) -> np.ndarray:
    """Active voxels of the seeded shell/plane union, raster order."""
    shells, planes = _draw_surfaces(G, n_shells, r_min, r_max, n_planes, seed)
    occ = np.zeros(G ** 3, dtype=bool)
    for c, r in shells:
        _mark_shell(occ, G, c, r)
    for nrm, p in planes:
        _mark_plane(occ, G, nrm, p)
    return linear_to_xyz(np.flatnonzero(occ), G)


def raster_coords(wl: Workload) -> np.ndarray:
    """The workload's active set in raster order (x slowest)."""
    P = wl.params
    if wl.kind == "uniform":
        c = uniform_coords(wl.grid, P["n"], wl.geom_seed)
        G = wl.grid
        lin = (c[:, 0].astype(np.int64) * G + c[:, 1]) * G + c[:, 2]
        return c[np.argsort(lin, kind="stable")]
    if wl.kind == "shell":
        return shell_coords(wl.grid, P["center"], P["radius"], P["half_width"])
    return surface_coords(wl.grid, P["n_shells"], P["r_min"], P["r_max"],
                          P["n_planes"], wl.geom_seed)


def geometry(wl: Workload, shuffle: bool = True) -> np.ndarray:
    """int32 (N,3) coordinates in caller order.

    uniform32 keeps its draw order; the others are raster-ordered and then
    shuffled with the workload's shuffle seed (or left raster-ordered when
    ``shuffle`` is False)."""
    if wl.kind == "uniform":
        return uniform_coords(wl.grid, wl.params["n"], wl.geom_seed)
    c = raster_coords(wl)
    if shuffle:
        perm = np.random.default_rng(wl.shuffle_seed).permutation(c.shape[0])
        c = c[perm]
    return np.ascontiguousarray(c, dtype=np.int32)


def values(wl: Workload, N: int, Ci: int | None = None, Co: int | None = None):
    """(feats, w, bias) as torch CPU tensors.

    feats (N,Ci) and w (K,Ci,Co) are float32 or bfloat16 (RNE from float32);
    bias (Co,) is float32."""
    import torch
    Ci = wl.Ci if Ci is None else Ci
    Co = wl.Co if Co is None else Co
    rng = np.random.default_rng(wl.value_seed)
    feats = rng.standard_normal((N, Ci), dtype=np.float32)
    w = rng.standard_normal((wl.K, Ci, Co), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(27.0 * Ci))
    bias = rng.standard_normal((Co,), dtype=np.float32) * np.float32(math.sqrt(0.1))
    tf = torch.from_numpy(feats)
    tw = torch.from_numpy(w)
    if wl.dtype == "bf16":
        tf = tf.to(torch.bfloat16)
        tw = tw.to(torch.bfloat16)
    return tf, tw, torch.from_numpy(bias)


def make(wl: Workload | str, shuffle: bool = True):
    """coords, feats, w, bias for a workload (CPU)."""
    if isinstance(wl, str):
        wl = by_name(wl)
    coords = geometry(wl, shuffle=shuffle)
    feats, w, bias = values(wl, coords.shape[0])
    return coords, feats, w, bias
