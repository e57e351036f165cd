"""Feature tensors of 4 GiB and more: the 64-bit row addressing paths.

Dense cubes whose bf16 feature tensor holds N * Ci * 2 >= 2^32 bytes:

* 256^3 sites, Ci = 128 (exactly 2^32 bytes).  Co = 64 runs the tile kernel
  (packed and unpacked entry points); a dense 8x8x4 Morton tile touches
  10x10x6 = 600 distinct rows, more than a tile's row list holds, so every
  tile takes the direct-gather path.  Co = 32 runs the register-gather kernel.
* 204^3 sites, Ci = 256 (4.35e9 bytes): the register-gather kernel.

The map's valid pairs have a closed form on a dense cube of side G with the
3x3x3 offsets: each axis contributes G + 2(G - 1) = 3G - 2 (offset 0 keeps G
sites, offsets -1 and +1 keep G - 1), so the count is (3G - 2)^3.  Map
columns and output rows are checked on a sample (random rows, the first and
last schedule tiles, the cube's corners); the oracle gets the needed feature
rows only, re-indexed.  Features come from torch's seeded device generator,
weights and bias from numpy's.
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


def dense_cube(G, seed):
    ax = np.arange(G, dtype=np.int32)
    c = np.stack(np.meshgrid(ax, ax, ax, indexing="ij"), -1).reshape(-1, 3)
    c = c[np.random.default_rng(seed).permutation(c.shape[0])]
    return np.ascontiguousarray(c, dtype=np.int32)


def sample_rows(coords, order, G, rng, n=1500):
    N = coords.shape[0]
    corners = np.flatnonzero(((coords == 0) | (coords == G - 1)).all(1))
    rows = np.concatenate([rng.choice(N, n, replace=False), order[:256], order[-256:], corners])
    return np.unique(rows.astype(np.int64))


def check_sampled(feats_dev, nb, w, bias, gpu_rows, tag):
    """nb: (K, nrows) oracle map columns (sentinel N)."""
    N = feats_dev.shape[0]
    need = np.unique(nb[nb != N])
    sub = feats_dev[torch.from_numpy(need).to(DEV)].cpu()
    local = np.where(nb != N, np.searchsorted(need, nb), need.shape[0]).astype(np.int32)
    ref, S = oracle.forward(sub, local, w, bias)
    rep = check_forward(gpu_rows, ref, S, bias.numpy(), "bf16")
    say(tag, rep)
    assert rep["fail"] == 0, rep


def weights(rng, K, Ci, Co):
    w = rng.standard_normal((K, Ci, Co), dtype=np.float32) * np.float32(1.0 / np.sqrt(27.0 * Ci))
    b = rng.standard_normal((Co,), dtype=np.float32) * np.float32(np.sqrt(0.1))
    return torch.from_numpy(w).to(torch.bfloat16), torch.from_numpy(b)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("G, Ci, Cos", [(256, 128, (64, 32)), (204, 256, (64,))],
                         ids=["cube256_ci128", "cube204_ci256"])
def test_forward_feats_over_4gib(G, Ci, Cos):
    N = G ** 3
    assert N * Ci * 2 >= 2 ** 32
    rng = np.random.default_rng(20261202 + G)
    coords = dense_cube(G, 7 + G)
    say(f"[large] G={G} N={N} Ci={Ci} Co={Cos}: building the map")
    nm = sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), 27, 1)
    assert nm.valid_pairs == (3 * G - 2) ** 3
    nbr, order = nm.export()
    torch.cuda.synchronize()
    rows = sample_rows(coords, order.cpu().numpy(), G, rng)
    nb = oracle.nmap_rows(coords, rows, 27, 1)
    g = nbr[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(g, nb)
    del nbr, order
    say(f"[large] G={G} map sample of {rows.shape[0]} columns bit-exact")

    gen = torch.Generator(device=DEV)
    gen.manual_seed(11 + G)
    feats = torch.randn((N, Ci), generator=gen, device=DEV, dtype=torch.bfloat16)
    rows_dev = torch.from_numpy(rows).to(DEV)
    for Co in Cos:
        w, bias = weights(rng, 27, Ci, Co)
        wd, bd = w.to(DEV), bias.to(DEV)
        outs = {"forward": sp.spconv_forward(feats, nm, wd, bd)}
        wp = sp.spconv_pack_weights(wd)
        if wp.numel():
            outs["forward_packed"] = sp.spconv_forward_packed(feats, nm, wd, wp, bd)
        torch.cuda.synchronize()
        for kind, out in outs.items():
            assert out.shape == (N, Co)
            got = out[rows_dev].float().cpu().numpy()
            check_sampled(feats, nb, w, bias, got, f"[large] G={G} Ci={Ci} Co={Co} {kind}")
        if len(outs) == 2:
            assert torch.equal(outs["forward"], outs["forward_packed"])
        del outs
