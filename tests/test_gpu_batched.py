"""Batched coordinates (spconv_build_nmap_batched): voxels are neighbours only
within one batch.  The reference is the oracle's map of each batch on its own,
stitched into the global numbering, so it shares nothing with the library's
slab placement of the batches.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_forward
import submanifold_sparse_convolution_spconv_amd as sp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stitched_nmap(coords4, K, d):
    """(K, N) map from per-batch oracle maps (sentinel N)."""
    N = coords4.shape[0]
    out = np.full((K, N), N, dtype=np.int32)
    for b in np.unique(coords4[:, 0]):
        idx = np.nonzero(coords4[:, 0] == b)[0]
        nb = oracle.nmap(np.ascontiguousarray(coords4[idx, 1:]), K, d)
        out[:, idx] = np.where(nb < idx.size, idx[np.minimum(nb, idx.size - 1)], N)
    return out


def batched_sites(rng, batches, G, density, edge_x=None):
    parts = []
    for b in range(batches):
        m = rng.random((G, G, G)) < density
        c = np.argwhere(m).astype(np.int64) - G // 2
        if edge_x is not None:        # voxels at the lowest and highest x a batch may use
            lo, hi = edge_x
            c = np.concatenate([c, [[lo, 0, 0], [lo, 1, 0], [hi, 0, 0], [hi, 0, 1]]])
            c = np.unique(c, axis=0)
        parts.append(np.concatenate([np.full((c.shape[0], 1), b), c], 1))
    c4 = np.concatenate(parts).astype(np.int32)
    return c4[rng.permutation(c4.shape[0])]


@pytest.mark.parametrize("batches,K,d", [(5, 27, 1), (3, 27, 2), (8, 125, 1), (1, 27, 1), (17, 27, 3)])
def test_batched_map_and_forward(batches, K, d):
    rng = np.random.default_rng(100 * batches + K + d)
    half = 1 << (20 - max(0, int(np.ceil(np.log2(batches)))))
    reach = d * (round(K ** (1 / 3)) - 1) // 2
    c4 = batched_sites(rng, batches, 12, 0.25, edge_x=(-half + reach, half - reach - 1))
    N = c4.shape[0]
    say(f"[batched] batches={batches} K={K} d={d} N={N}")
    nm = sp.spconv_build_nmap_batched(torch.from_numpy(c4).to(DEV), batches, K, d)
    nbr, order = nm.export()
    torch.cuda.synchronize()
    ref = stitched_nmap(c4, K, d)
    assert np.array_equal(nbr.cpu().numpy(), ref)
    assert nm.valid_pairs == int((ref != N).sum())
    o = order.cpu().numpy()
    assert np.array_equal(np.sort(o), np.arange(N))
    Ci, Co = 64, 32
    feats = torch.from_numpy(rng.standard_normal((N, Ci)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((K, Ci, Co)) / 30).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32))
    out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV))
    r, S = oracle.forward(feats, ref, w, bias)
    rep = check_forward(out.float().cpu().numpy(), r, S, bias.numpy(), "bf16")
    say("[batched]", rep)
    assert rep["fail"] == 0


def test_batched_range_errors():
    B = 4
    half = 1 << (20 - 2)
    ok = np.array([[0, 0, 0, 0], [3, half - 2, 5, -7]], dtype=np.int32)
    sp.spconv_build_nmap_batched(torch.from_numpy(ok).to(DEV), B, 27, 1)
    for bad in ([4, 0, 0, 0], [-1, 0, 0, 0], [1, half - 1, 0, 0], [2, -half, 0, 0], [0, 0, 1 << 20, 0]):
        c = torch.from_numpy(np.array([[0, 0, 0, 0], bad], dtype=np.int32)).to(DEV)
        with pytest.raises(sp.SpconvError) as e:
            sp.spconv_build_nmap_batched(c, B, 27, 1)
        assert e.value.code == -3, bad
    dup = torch.from_numpy(np.array([[1, 2, 3, 4], [0, 2, 3, 4], [1, 2, 3, 4]], dtype=np.int32)).to(DEV)
    with pytest.raises(sp.SpconvError) as e:
        sp.spconv_build_nmap_batched(dup, B, 27, 1)
    assert e.value.code == -4
