"""The seeded input recipes: realised sizes, pruned surface enumeration, values."""
import numpy as np
import pytest
import torch

import workloads as W

# realised voxel counts of the five recipes (the generator's own self-check)
EXPECTED_N = {"uniform32": 4096, "shell64": 29578, "surf256": 1006716,
              "surf512d2": 2177577, "surf1024": 10963210}


@pytest.mark.parametrize("name", ["uniform32", "shell64", "surf256", "surf512d2", "surf1024"])
def test_realised_sizes(name):
    wl = W.by_name(name)
    c = W.geometry(wl)
    assert c.dtype == np.int32 and c.shape == (EXPECTED_N[name], 3)
    assert c.min() >= 0 and c.max() < wl.grid
    lin = (c[:, 0].astype(np.int64) * wl.grid + c[:, 1]) * wl.grid + c[:, 2]
    assert np.unique(lin).size == lin.size


@pytest.mark.parametrize("seed", range(4))
def test_pruned_surfaces_equal_dense(seed):
    G = 56
    shells, planes = W._draw_surfaces(G, 5, 3.0, 30.0, 4, seed)
    dense = np.flatnonzero(W.dense_surface_mask(G, shells, planes).ravel())
    c = W.surface_coords(G, 5, 3.0, 30.0, 4, seed)
    lin = (c[:, 0].astype(np.int64) * G + c[:, 1]) * G + c[:, 2]
    assert np.array_equal(lin, dense)


def test_shuffle_is_permutation_of_raster():
    wl = W.by_name("shell64")
    a = W.geometry(wl, shuffle=False)
    b = W.geometry(wl, shuffle=True)
    ka = np.sort((a[:, 0].astype(np.int64) * 64 + a[:, 1]) * 64 + a[:, 2])
    kb = np.sort((b[:, 0].astype(np.int64) * 64 + b[:, 1]) * 64 + b[:, 2])
    assert np.array_equal(ka, kb) and not np.array_equal(a, b)


def test_values_dtypes_and_scale():
    wl = W.by_name("shell64")
    f, w, b = W.values(wl, 20000)
    assert f.dtype == torch.bfloat16 and w.dtype == torch.bfloat16 and b.dtype == torch.float32
    assert f.shape == (20000, 64) and w.shape == (27, 64, 64) and b.shape == (64,)
    assert abs(f.float().std().item() - 1.0) < 0.02
    assert abs(w.float().var().item() * 27 * 64 - 1.0) < 0.05
    f2, w2, b2 = W.values(wl, 20000)
    assert torch.equal(f, f2) and torch.equal(w, w2) and torch.equal(b, b2)
    wl1 = W.by_name("uniform32")
    f, w, b = W.values(wl1, 4096)
    assert f.dtype == torch.float32 and w.shape == (27, 32, 32)
