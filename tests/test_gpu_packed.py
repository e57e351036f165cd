"""GPU tests of the packed-weight path (spconv_pack_weights /
spconv_forward_packed): the packed buffer against its documented layouts,
restated here in numpy, and the packed forward against the unpacked one (bit
for bit: the unpacked entry point packs w itself and runs the same kernel)
and against the oracle."""
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


def tile_width(Ci, Co):
    """Output-channel tile of the LDS-staged kernel: 128, 64 or 32 (the largest
    dividing Co), at most 64 for Ci = 256."""
    bn = 128 if Co % 128 == 0 else 64 if Co % 64 == 0 else 32
    return min(bn, 64) if Ci == 256 else bn


def reference_pack_frag(w):
    """Fragment order (Ci = 128, Co % 64 == 0): 16-byte unit
    e = (((k (Co/64) + c) 4 + s) 4 + j) 64 + l, lane l = m + 16 q, holds
    w[k, 32s + 8q : 32s + 8q + 8, 64c + 16 (m // 4) + 4j + m % 4]."""
    K, Ci, Co = w.shape
    u16 = w.view(torch.int16).cpu().numpy().view(np.uint16)
    ncg = Co // 64
    out = np.zeros((K, ncg, 4, 4, 64, 8), np.uint16)
    l = np.arange(64)
    m, q = l % 16, l // 16
    for c in range(ncg):
        for s_ in range(4):
            for j in range(4):
                co = 64 * c + 16 * (m // 4) + 4 * j + m % 4              # (64,)
                ci = 32 * s_ + 8 * q[:, None] + np.arange(8)[None, :]    # (64, 8)
                out[:, c, s_, j] = u16[:, ci, co[:, None]]
    return out.reshape(-1).view(np.uint8)


def reference_pack(w):
    """Packed layout, unit by unit: slice (k, tile) holds Ci/8 planes of
    BN rows of 16 bytes; row r = 16j + m of plane u carries
    w[k, 8u:8u+8, tile*BN + co(j, m)], co(j, m) = (m//4)*4NJ + 4j + m%4, and
    is stored at row r XOR 16 in odd planes."""
    K, Ci, Co = w.shape
    bn = tile_width(Ci, Co)
    nj = bn // 16
    u16 = w.view(torch.int16).cpu().numpy().view(np.uint16)
    out = np.zeros((K, Co // bn, Ci // 8, bn, 8), np.uint16)
    r = np.arange(bn)
    j, m = r // 16, r % 16
    co_loc = (m // 4) * 4 * nj + 4 * j + m % 4
    for t in range(Co // bn):
        cols = t * bn + co_loc                                   # (bn,)
        blk = u16[:, :, cols]                                    # (K, Ci, bn)
        out[:, t] = blk.reshape(K, Ci // 8, 8, bn).transpose(0, 1, 3, 2)
    out[:, :, 1::2] = out[:, :, 1::2][:, :, :, r ^ 16]          # stored row p holds logical row p ^ 16
    return out.reshape(-1).view(np.uint8)


def frag_order(Ci, Co):
    return Ci == 128 and Co % 64 == 0


@pytest.mark.parametrize("shape", [(27, 128, 128), (3, 128, 64), (2, 128, 192), (3, 128, 96), (2, 256, 64),
                                   (2, 256, 96), (2, 128, 32), (1, 256, 256)])
def test_pack_layout(shape):
    K, Ci, Co = shape
    say(f"[pack] K={K} Ci={Ci} Co={Co}")
    g = torch.Generator().manual_seed(K * 1000 + Ci + Co)
    w = torch.randn(K, Ci, Co, generator=g).to(torch.bfloat16)
    n = sp.spconv_pack_weights_size(K, Ci, Co, sp.SPCONV_BF16)
    bn = tile_width(Ci, Co)
    assert n == K * Ci * Co * 2          # w's own size: no padding rows
    wp = sp.spconv_pack_weights(w.to(DEV))
    torch.cuda.synchronize()
    assert wp.numel() == n
    ref = reference_pack_frag(w) if frag_order(Ci, Co) else reference_pack(w)
    assert np.array_equal(wp.cpu().numpy(), ref)


def test_pack_empty_where_no_packed_form():
    for (Ci, Co, dt) in [(128, 128, sp.SPCONV_F32), (64, 64, sp.SPCONV_BF16), (32, 96, sp.SPCONV_BF16)]:
        assert sp.spconv_pack_weights_size(27, Ci, Co, dt) == 0
    # the packed forward then equals the plain one with an empty pack
    rng = np.random.default_rng(5)
    coords = np.argwhere(rng.random((9, 9, 9)) < 0.3).astype(np.int32)
    N = coords.shape[0]
    feats = torch.from_numpy(rng.standard_normal((N, 64)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy(rng.standard_normal((27, 64, 64)).astype(np.float32) / 40).to(torch.bfloat16).to(DEV)
    nm = sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), 27, 1)
    wp = sp.spconv_pack_weights(w)
    a = sp.spconv_forward(feats, nm, w)
    b = sp.spconv_forward_packed(feats, nm, w, wp)
    torch.cuda.synchronize()
    assert wp.numel() == 0
    assert torch.equal(a, b)


def _check_sampled(coords, feats, w, bias, out, rows, K, d, tag):
    nb = oracle.nmap_rows(coords, rows, K, d)
    ref, S = oracle.forward(feats, nb, w, bias)
    g = out[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    rep = check_forward(g, ref, S, bias.numpy(), "bf16")
    say(tag, rep)
    assert rep["fail"] == 0, rep


@pytest.mark.parametrize("name", ["surf256", "surf1024"])
def test_forward_packed_full_size(name):
    wl = W.by_name(name)
    coords = W.geometry(wl)
    N = coords.shape[0]
    feats, w, bias = W.values(wl, N)
    say(f"[packed] {name} N={N} Ci={wl.Ci} Co={wl.Co}")
    nm = sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), wl.K, wl.dilation)
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    wp = sp.spconv_pack_weights(wd)
    a = sp.spconv_forward(fd, nm, wd, bd)
    b = sp.spconv_forward_packed(fd, nm, wd, wp, bd)
    b2 = sp.spconv_forward_packed(fd, nm, wd, wp, bd)
    torch.cuda.synchronize()
    assert wp.numel() > 0
    assert torch.equal(a, b), "packed and unpacked forwards differ"
    assert torch.equal(b, b2), "packed forward not deterministic"
    # every row of the packed and the unpacked forward against the oracle:
    # test_gpu_parity.test_forward_every_row_full_size


@pytest.mark.parametrize("case", [(11, 0.4, 27, 1, 256, 32), (12, 0.3, 27, 1, 256, 96),
                                  (16, 0.08, 27, 3, 128, 64), (10, 0.3, 125, 1, 128, 160)],
                         ids=lambda c: "G%d_K%d_%dx%d" % (c[0], c[2], c[4], c[5]))
def test_forward_packed_small(case):
    G, dens, K, d, Ci, Co = case
    rng = np.random.default_rng(G + K + Ci + Co)
    coords = np.argwhere(rng.random((G, G, G)) < dens).astype(np.int32) - 4
    coords = coords[rng.permutation(coords.shape[0])]
    N = coords.shape[0]
    say(f"[packed-small] N={N} K={K} d={d} Ci={Ci} Co={Co}")
    feats = torch.from_numpy(rng.standard_normal((N, Ci)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((K, Ci, Co)) / np.sqrt(K * Ci)).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32))
    nm = sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), K, d)
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    wp = sp.spconv_pack_weights(wd)
    a = sp.spconv_forward(fd, nm, wd, bd)
    b = sp.spconv_forward_packed(fd, nm, wd, wp, bd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    _check_sampled(coords, feats, w, bias, b, np.arange(N), K, d, "[packed-small]")


def _packed_vs_unpacked_and_oracle(coords, nb, K, d, Co, tag, wrap=False):
    rng = np.random.default_rng(1234 + K + Co + coords.shape[0])
    N = coords.shape[0] if coords is not None else nb.shape[1]
    feats = torch.from_numpy(rng.standard_normal((N, 128)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((K, 128, Co)) / np.sqrt(K * 128)).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32))
    if wrap:
        nm = sp.spconv_nmap_wrap(torch.from_numpy(nb).to(DEV))
    else:
        nm = sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), K, d)
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    a = sp.spconv_forward(fd, nm, wd, bd)
    b = sp.spconv_forward_packed(fd, nm, wd, sp.spconv_pack_weights(wd), bd)
    torch.cuda.synchronize()
    assert torch.equal(a, b), tag
    ref, S = oracle.forward(feats, nb, w, bias)
    rep = check_forward(b.float().cpu().numpy(), ref, S, bias.numpy(), "bf16")
    say(tag, rep)
    assert rep["fail"] == 0, rep


@pytest.mark.parametrize("N", [1, 2, 255, 256, 257, 511, 767])
def test_packed_ragged_sizes(N):
    """Ci = 128 (the tile kernel over distinct rows): one partial tile, exact
    tiles and ragged tails."""
    rng = np.random.default_rng(N)
    cells = np.argwhere(np.ones((12, 12, 12), bool)).astype(np.int32)
    coords = cells[rng.choice(cells.shape[0], N, replace=False)]
    _packed_vs_unpacked_and_oracle(coords, oracle.nmap(coords, 27, 1), 27, 1, 128, f"[packed-ragged] N={N}")


def test_packed_k1_and_all_sentinel():
    rng = np.random.default_rng(8)
    coords = np.argwhere(rng.random((10, 10, 10)) < 0.5).astype(np.int32)
    N = coords.shape[0]
    # K = 1: one offset (the centre) per tile
    _packed_vs_unpacked_and_oracle(coords, oracle.nmap(coords, 1, 1), 1, 1, 128, "[packed-k1]")
    # a wrapped map with no present neighbour: every block inactive, the output is the bias
    nb = np.full((27, N), N, dtype=np.int32)
    _packed_vs_unpacked_and_oracle(coords, nb, 27, 1, 64, "[packed-sentinel]", wrap=True)


@pytest.mark.parametrize("K,N", [(343, 70000), (729, 4000), (27, 33 * 256 + 17), (27, 300 * 256 + 5)])
def test_packed_tiles_per_workgroup(K, N):
    """The Ci = 128 tile kernel's persistent workgroups (one per CU, each
    XCD's run of tiles dealt round-robin): maps of more than 27 offsets have no
    distinct-row lists and run every tile in its direct form (two offsets'
    rows staged at a time); tile counts below, at and above the CU count and
    not a multiple of 8.  Packed equals unpacked bit for bit; sampled rows
    against the oracle."""
    rng = np.random.default_rng(K + N)
    side = max(28, int(np.ceil((2.5 * N) ** (1 / 3))))
    cells = np.argwhere(np.ones((side, side, side), bool)).astype(np.int32) - 10
    coords = cells[rng.choice(cells.shape[0], N, replace=False)]
    say(f"[packed-tpw] K={K} N={N} tiles={(N + 255) // 256}")
    feats = torch.from_numpy(rng.standard_normal((N, 128)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((K, 128, 64)) / np.sqrt(K * 128)).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(64).astype(np.float32))
    nm = sp.spconv_build_nmap(torch.from_numpy(coords).to(DEV), K, 1)
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    a = sp.spconv_forward(fd, nm, wd, bd)
    b = sp.spconv_forward_packed(fd, nm, wd, sp.spconv_pack_weights(wd), bd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    rows = np.unique(np.concatenate([rng.choice(N, 300, replace=False), [0, N - 1]]))
    _check_sampled(coords, feats, w, bias, b, rows, K, 1, "[packed-tpw]")


def test_packed_two_pass_and_direct_tiles():
    """The tile kernel's three ways of running a 128-row tile: one staging
    pass (a sparse shell: at most 315 distinct neighbour rows), three passes
    of one x-offset layer each (a dense block: a 4x4x8 Morton tile has
    6x6x10 = 360 distinct rows, a layer 4x6x10 = 240), and the direct form (a
    dense block at dilation 4: 12x12x16 = 2304 distinct rows, a layer 4x12x16
    = 768).  Every output row against the oracle, packed equal to unpacked.
    The maps have more than 65536 rows, so that the tile kernel runs."""
    rng = np.random.default_rng(77)
    dense = np.argwhere(np.ones((24, 24, 24), bool)).astype(np.int32)
    g = np.argwhere(np.ones((128, 128, 128), bool)).astype(np.int32) - 64
    r = np.sqrt((g.astype(np.float64) ** 2).sum(1))
    shell = g[np.abs(r - 60) < 0.8] + np.array([100, 0, 0], np.int32)
    mixed = np.concatenate([dense, shell])
    assert mixed.shape[0] > 65536
    mixed = mixed[rng.permutation(mixed.shape[0])]
    _packed_vs_unpacked_and_oracle(mixed, oracle.nmap(mixed, 27, 1), 27, 1, 128, "[packed-passes] mixed")
    big = np.argwhere(np.ones((44, 44, 44), bool)).astype(np.int32)
    assert big.shape[0] > 65536
    _packed_vs_unpacked_and_oracle(big, oracle.nmap(big, 27, 4), 27, 4, 64, "[packed-passes] direct")


def test_tile_queue_counters_reused():
    """The tile kernel takes tiles from per-launch counters that every launch
    leaves at zero for the next user of its slots: more launches than there
    are slots (8192), with more tiles than workgroups, all give the first
    launch's output bit for bit."""
    rng = np.random.default_rng(5)
    cells = np.argwhere(rng.random((64, 64, 64)) < 0.35).astype(np.int32)
    N = cells.shape[0]
    assert (N + 127) // 128 > 2 * 256
    feats = torch.from_numpy(rng.standard_normal((N, 128)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy((rng.standard_normal((27, 128, 128)) / 60).astype(np.float32)).to(torch.bfloat16).to(DEV)
    bias = torch.from_numpy(rng.standard_normal(128).astype(np.float32)).to(DEV)
    nm = sp.spconv_build_nmap(torch.from_numpy(cells).to(DEV), 27, 1)
    wp = sp.spconv_pack_weights(w)
    first = sp.spconv_forward_packed(feats, nm, w, wp, bias)
    out = torch.empty_like(first)
    for i in range(8300):
        sp.spconv_forward_packed(feats, nm, w, wp, bias, out=out)
        if i % 1000 == 999:
            torch.cuda.synchronize()
            assert torch.equal(out, first), i
    torch.cuda.synchronize()
    assert torch.equal(out, first)
    say(f"[queue] N={N} 8300 launches equal to the first")
