"""One GPU's share of a spatial split: the voxels are cut into Morton ranges
balanced by valid pairs; a shard holds its own rows plus their halo (the
neighbours owned by other ranges), appended after the own rows.  Built and
convolved on its own, the shard's own rows must give exactly the outputs of
the whole cloud's forward (every own row sees its full neighbourhood, and the
kernel's per-row summation order does not depend on where the row lands), and
match the oracle on sampled rows.  Morton order, ranges and halos come from
the oracle's codes and map.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.compare import check_forward
import submanifold_sparse_convolution_spconv_amd as sp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def morton_shards(coords, nb, parts):
    """Own rows (caller indices) of each Morton range, balanced by valid pairs."""
    N = coords.shape[0]
    order = np.argsort(oracle.morton(coords), kind="stable")
    cum = np.cumsum((nb != N).sum(0)[order])
    cuts = [0] + [int(np.searchsorted(cum, cum[-1] * i // parts)) for i in range(1, parts)] + [N]
    return [order[a:b] for a, b in zip(cuts[:-1], cuts[1:])]


@pytest.mark.parametrize("name,parts", [("surf256", 4), ("surf512d2", 2)])
def test_shard_equals_whole_cloud(name, parts):
    wl = W.by_name(name)
    coords = W.geometry(wl)
    N = coords.shape[0]
    feats, w, bias = W.values(wl, N)
    nb = oracle.nmap(coords, wl.K, wl.dilation)
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    say(f"[shard] {name} N={N} parts={parts}")
    whole = sp.spconv_forward(fd, sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), wl.K, wl.dilation), wd, bd)
    rng = np.random.default_rng(60 + wl.index)
    for s, own in enumerate(morton_shards(coords, nb, parts)):
        inside = np.zeros(N + 1, dtype=bool)
        inside[own] = True
        inside[N] = True
        cols = nb[:, own].reshape(-1)
        halo = np.unique(cols[~inside[cols]])
        rows = np.concatenate([own, halo])
        say(f"[shard] {name} shard {s}: own={own.size} halo={halo.size} ({halo.size / own.size:.3%})")
        c_s = torch.from_numpy(np.ascontiguousarray(coords[rows])).to(DEV)
        nm_s = sp.spconv_build_nmap(c_s, wl.K, wl.dilation)
        out_s = sp.spconv_forward(fd[torch.from_numpy(rows).to(DEV)].contiguous(), nm_s, wd, bd)
        # own rows: identical to the whole cloud's outputs
        mine = out_s[:own.size]
        ref_whole = whole[torch.from_numpy(own).to(DEV)]
        assert torch.equal(mine, ref_whole), f"shard {s}"
        # and within tolerance of the oracle on sampled own rows
        pick = np.sort(rng.choice(own.size, min(1000, own.size), replace=False))
        ref, S = oracle.forward(feats, nb[:, own[pick]], w, bias)
        rep = check_forward(mine[torch.from_numpy(pick).to(DEV)].float().cpu().numpy(), ref, S, bias.numpy(),
                            wl.dtype)
        assert rep["fail"] == 0, rep
        # the shard's map, read in shard numbering, is the whole map restricted to own rows
        nbr_s, _ = nm_s.export()
        to_global = np.append(rows, N)
        got = to_global[nbr_s[:, :own.size].cpu().numpy()]
        assert np.array_equal(got, nb[:, own])
